"""The no-allocation entry point (sv_verify_sample_batched_noalloc) on the
GPU, through the C ABI: its outputs and row statistics equal those of
sv_verify_sample_batched (the same kernels on a caller's workspace) and the
oracle's, on consecutive calls of decreasing size that share the library's
static scratch; sizes beyond the scratch are refused."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import speculative_decoding_verification_row_amd as sv

from _parity import check_sampled

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(msg):
    print(f"\n[gpu case] {msg}", flush=True)


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    sv.load_library()
    yield
    torch.cuda.synchronize()


def _inputs(B, K, V, seed):
    b = workloads.make_batch("c3", B, K, V, seed=seed)
    host = (b.target_probs, b.draft_probs, b.draft_tokens, b.uniforms)
    return host, [torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in host]


def test_noalloc_matches_workspace_call_on_calls_of_decreasing_size():
    # B=64 K=5 V=128256 takes the walks, B=3 K=4 V=20011 one block per draft
    # row, B=9 K=7 V=4099 walks again over what the two before left behind
    for j, (B, K, V) in enumerate([(64, 5, 128256), (3, 4, 20011), (9, 7, 4099)]):
        _case(f"no-allocation call {j}: B={B} K={K} V={V}")
        host, (tp, dp, dt, u) = _inputs(B, K, V, seed=40 + j)
        n0 = torch.empty(B, dtype=torch.int32, device=DEV)
        x0 = torch.empty(B, dtype=torch.int32, device=DEV)
        st0 = torch.empty((B, K + 1, 48), dtype=torch.uint8, device=DEV)
        sv.sv_verify_sample_batched_noalloc(tp, dp, dt, u, n0, x0, stats=st0)
        n1 = torch.empty_like(n0)
        x1 = torch.empty_like(x0)
        sv.sv_verify_sample_batched_noalloc(tp, dp, dt, u, n1, x1)    # no statistics
        ws = torch.empty(sv.sv_workspace_size(B, K, V, True), dtype=torch.uint8, device=DEV)
        sv.sv_workspace_init(ws)
        rn, rx, rst = sv.sv_verify_sample_batched(tp, dp, dt, u, workspace=ws, stats=True)
        torch.cuda.synchronize()
        for a, b in ((n0, rn), (x0, rx), (st0, rst), (n1, rn), (x1, rx)):
            assert torch.equal(a, b)
        check_sampled(n0.cpu().numpy(), x0.cpu().numpy(), sv.stats_to_numpy(st0), oracle.verify_sample(*host))


def test_noalloc_refuses_sizes_beyond_the_scratch():
    _case("no-allocation call: workspace beyond SV_SCRATCH_BYTES is refused")
    B, K, V = 1024, 16, 128256
    assert sv.sv_workspace_size(B, K, V, True) > sv.SV_SCRATCH_BYTES
    # operands of these shapes would take 8.9 GB; the library refuses on the
    # sizes before it reads any buffer or launches anything, so one small
    # allocation stands in for every pointer
    base = torch.zeros(1, dtype=torch.float32, device=DEV)
    lib = sv.load_library()
    rc = lib.sv_verify_sample_batched_noalloc(base.data_ptr(), base.data_ptr(), base.data_ptr(), base.data_ptr(),
                                              B, K, V, base.data_ptr(), base.data_ptr(), None, None)
    assert rc == sv.SV_ERR_SCRATCH
