"""GPU parity of the early-exit entry point (sv_verify_sample_early_batched):
its outputs are those of sv_verify_sample_batched bit for bit (the same
decisions from the same published partials; only rows no reader needs go
unread), and so the fp64 oracle's, to the sampled bar.  Small and ragged
shapes in both forms of the pass, seeded random shapes, the forced
recompute path, and the B=256 K=5 V=128256 workload."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads.device import device_batch
import speculative_decoding_verification_row_amd as sv

from _parity import check_sampled
from test_gpu_parity import SMALL, _random_rows
from test_gpu_random_shapes import _shape, _rows
from _forms import FORMS, set_form

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


@pytest.fixture(params=FORMS)
def form(request, monkeypatch):
    set_form(monkeypatch, request.param)
    return request.param


def _both(tp, dp, dt, u):
    """(early n, early next, full n, full next) as numpy, each call on its own
    fresh workspace."""
    B, K1, V = tp.shape
    out = []
    for f in (sv.sv_verify_sample_early_batched, sv.sv_verify_sample_batched):
        ws = torch.empty(sv.sv_workspace_size(B, K1 - 1, V, True), dtype=torch.uint8, device=DEV)
        sv.sv_workspace_init(ws)
        n, nx = f(tp, dp, dt, u, workspace=ws)
        torch.cuda.synchronize()
        out += [n.cpu().numpy(), nx.cpu().numpy()]
        assert sv.sv_workspace_error(ws) == 0
    return out


def _dev(*arrays):
    return [torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in arrays]


@pytest.mark.parametrize("B,K,V", SMALL, ids=lambda x: str(x))
def test_early_small(B, K, V, form):
    _case(f"early exit small B={B} K={K} V={V} form={form}")
    p, q, t, u = _random_rows(np.random.default_rng(B * 1000 + K * 10 + V), B, K, V)
    en, ex, fn, fx = _both(*_dev(p, q, t, u))
    assert np.array_equal(en, fn) and np.array_equal(ex, fx)
    check_sampled(en, ex, None, oracle.verify_sample(p, q, t, u))


@pytest.mark.parametrize("j", range(12))
def test_early_random_shapes(j):
    B, K, V, rng = _shape(j)
    _case(f"early exit random shape {j}: B={B} K={K} V={V}")
    p, q, t, u = _rows(rng, B, K, V)
    en, ex, fn, fx = _both(*_dev(p, q, t, u))
    assert np.array_equal(en, fn) and np.array_equal(ex, fx)
    check_sampled(en, ex, None, oracle.verify_sample(p, q, t, u))


def test_early_forced_recompute(monkeypatch):
    """With every partial recomputed by its reader, the bonus blocks never
    skip (the outcome word is not trusted then) and the outputs still match."""
    monkeypatch.setenv("SV_VERIFY_FORCE_RECOMPUTE", "1")
    _case("early exit with forced recompute B=6 K=5 V=40000")
    p, q, t, u = _random_rows(np.random.default_rng(5), 6, 5, 40000)
    en, ex, fn, fx = _both(*_dev(p, q, t, u))
    assert np.array_equal(en, fn) and np.array_equal(ex, fx)
    check_sampled(en, ex, None, oracle.verify_sample(p, q, t, u))


def test_early_full_workload():
    """B=256 K=5 V=128256 (the synthetic mix of the benchmark), two input
    sets in turn on one workspace: every output equal to the full pass's."""
    c = dict(workloads.CONFIGS[3])
    B, K, V = c["B"], c["K"], c["V"]
    _case(f"early exit full workload B={B} K={K} V={V} (generating)")
    sets = [device_batch(c["family"], B, K, V, seed=s, device=DEV, sampled=True) for s in range(2)]
    ws = torch.empty(sv.sv_workspace_size(B, K, V, True), dtype=torch.uint8, device=DEV)
    sv.sv_workspace_init(ws)
    for rep in range(4):
        db = sets[rep % 2]
        n, nx = sv.sv_verify_sample_batched(db["tp"], db["dp"], db["dt"], db["u"], workspace=ws)
        en, ex = sv.sv_verify_sample_early_batched(db["tp"], db["dp"], db["dt"], db["u"], workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(en, n) and torch.equal(ex, nx), rep
    assert 0 < int((n < K).sum()) < B
    assert sv.sv_workspace_error(ws) == 0
    del sets
    torch.cuda.empty_cache()


@pytest.mark.parametrize("tau", [0.5, 1.0, 0.02])
@pytest.mark.parametrize("B,K,V", [(5, 4, 1000), (3, 3, 1003), (2, 5, 40001), (3, 9, 5000)],
                         ids=lambda x: str(x))
def test_early_logits(B, K, V, tau, form):
    """The logits early exit: outputs equal to the full logits pass's, bit
    for bit, and to the logits oracle's to the sampled bar."""
    from test_gpu_logits import _rows as logit_rows, check
    from oracle.logits import verify_sample_logits
    _case(f"early exit logits B={B} K={K} V={V} tau={tau} form={form}")
    lp, lq, t, u = logit_rows(np.random.default_rng(B * 31 + K + V), B, K, V, tau)
    tl, dl, dt, ud = _dev(lp, lq, t, u)
    out = []
    for f in (sv.sv_verify_sample_logits_early_batched, sv.sv_verify_sample_logits_batched):
        ws = torch.empty(sv.sv_workspace_size(B, K, V, True), dtype=torch.uint8, device=DEV)
        sv.sv_workspace_init(ws)
        n, nx = f(tl, dl, dt, ud, tau, workspace=ws)
        torch.cuda.synchronize()
        out += [n.cpu().numpy(), nx.cpu().numpy()]
    assert np.array_equal(out[0], out[2]) and np.array_equal(out[1], out[3])
    check(out[0], out[1], verify_sample_logits(lp, lq, t, u, tau))


def test_early_logits_full_workload():
    """B=256 K=5 V=128256 logits (the synthetic mix), tau = 1, four calls on
    one workspace over two input sets: every output equal to the full
    logits pass's."""
    c = dict(workloads.CONFIGS[3])
    B, K, V = c["B"], c["K"], c["V"]
    _case(f"early exit logits full workload B={B} K={K} V={V} (generating)")
    sets = [device_batch(c["family"], B, K, V, seed=s, device=DEV, sampled=True, logits=True) for s in range(2)]
    ws = torch.empty(sv.sv_workspace_size(B, K, V, True), dtype=torch.uint8, device=DEV)
    sv.sv_workspace_init(ws)
    for rep in range(4):
        db = sets[rep % 2]
        n, nx = sv.sv_verify_sample_logits_batched(db["tp"], db["dp"], db["dt"], db["u"], 1.0, workspace=ws)
        en, ex = sv.sv_verify_sample_logits_early_batched(db["tp"], db["dp"], db["dt"], db["u"], 1.0, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(en, n) and torch.equal(ex, nx), rep
    assert 0 < int((n < K).sum()) < B
    del sets
    torch.cuda.empty_cache()
