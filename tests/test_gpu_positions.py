"""GPU parity of a rejection planted at every draft position in turn, through
the C ABI, in both forms of the pass and every sampled entry point, against
the fp64 oracles.

A walk takes its rows two steps a turn (the logits walk alternates its two
row buffers), leaves its search at the first rejected row, and streams or
stops after it; these cases make it leave at every step of a turn, for odd
and even K.  Sequence s of a batch of K + 1 sequences: draft rows 0..s-1
equal their target rows and carry the token at the row's largest value, so
they accept whatever u < 1 is drawn (q(t) P = p(t) Q exactly); row s (s < K)
carries a token outside [0, V), which every reading rejects; the rows after
s are the workload's own.  So n = s, and sequence K accepts every draft.
Draft row s is the workload's, not a copy of its target row, so the draw at
n = s is from a residual with mass (the spec-verify kernel card, section
"Method").
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.logits import verify_sample_logits
import speculative_decoding_verification_row_amd as sv

from _parity import check_logits, check_sampled
from _forms import FORMS, set_form

pytestmark = pytest.mark.gpu
DEV = "cuda"
SHAPES = [(6, 9000), (7, 9000), (6, 40001), (7, 130)]


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


def _planted(K, V, seed, logits):
    B = K + 1
    b = workloads.make_batch("c3", B, K, V, seed=seed, logits=logits)
    p, q = b.target_probs.copy(), b.draft_probs.copy()
    t, u = b.draft_tokens.copy(), b.uniforms.copy()
    for s in range(B):
        for i in range(min(s, K)):
            q[s, i] = p[s, i]
            t[s, i] = int(np.argmax(p[s, i]))
        if s < K:
            t[s, s] = V + 5
    assert np.all(u < 1.0)
    return p, q, t, u, np.arange(B)


def _dev(*arrays):
    return [torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in arrays]


def _np(*ts):
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in ts]


@pytest.mark.parametrize("K,V", SHAPES, ids=lambda x: str(x))
def test_rejection_at_each_position_probabilities(K, V, form):
    _case(f"rejection at each position, probabilities K={K} V={V} form={form}")
    p, q, t, u, n_want = _planted(K, V, seed=17 * K + V, logits=False)
    o = oracle.verify_sample(p, q, t, u)
    assert np.array_equal(o["n_accepted"], n_want)
    args = _dev(p, q, t, u)
    n, nx, st = sv.sv_verify_sample_batched(*args, stats=True)
    n, nx = _np(n, nx)
    assert np.array_equal(n, n_want)
    rep = check_sampled(n, nx, sv.stats_to_numpy(st), o)
    for name, (a, b_) in {"plain": sv.sv_verify_sample_batched(*args),
                          "early": sv.sv_verify_sample_early_batched(*args)}.items():
        a, b_ = _np(a, b_)
        assert np.array_equal(a, n) and np.array_equal(b_, nx), name
    print(f"  parity {rep}")


@pytest.mark.parametrize("tau", [1.0, 0.7])
@pytest.mark.parametrize("K,V", SHAPES, ids=lambda x: str(x))
def test_rejection_at_each_position_logits(K, V, tau, form):
    _case(f"rejection at each position, logits K={K} V={V} tau={tau} form={form}")
    tl, dl, t, u, n_want = _planted(K, V, seed=19 * K + V, logits=True)
    o = verify_sample_logits(tl, dl, t, u, tau)
    assert np.array_equal(o["n_accepted"], n_want)
    args = _dev(tl, dl, t, u)
    n, nx = _np(*sv.sv_verify_sample_logits_batched(*args, tau))
    assert np.array_equal(n, n_want)
    rep = check_logits(n, nx, o)
    ne, nxe = _np(*sv.sv_verify_sample_logits_early_batched(*args, tau))
    assert np.array_equal(ne, n) and np.array_equal(nxe, nx)
    print(f"  parity {rep}")
