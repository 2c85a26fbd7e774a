"""GPU parity of the two rarely taken paths of the sampled passes, through
the C ABI, in both forms of the pass (walks, one block per draft row) and
every sampled entry point (probabilities with and without row statistics, early exit,
logits, logits with early exit).

1. The zero-residual fallback (R8; the spec-verify kernel card, section
   "Method": the residual is norm(max(0, p - q))).  A rejected draft row whose
   residual has no mass draws from its target row p_n.  Planted exactly:
   draft row n equal to target row n bit for bit (or, on probabilities, twice
   it), and a rejected token that lies outside [0, V) or has p(t) = q(t) = 0;
   rows before n accept with certainty (q = p, a token with p(t) > 0), so
   n = 0 and n in mid-draft both occur.  The oracle's draw kind is 3 there,
   and every output must equal the oracle's.
2. Decisions that give up.  A walk (or row block) decides each row from its
   siblings' published partials and, when they do not arrive in time, leaves
   the decision to the block that finishes the sequence, which decides from
   the partials it gathers.  SV_VERIFY_FORCE_LOST=1 makes every such in-pass
   decision give up while the finishing blocks still trust the published
   words, so the outputs rest on every row's partial as the walks published
   it after losing their decision.  Outputs must equal those of the same
   call without the hook, and the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.logits import verify_sample_logits
import speculative_decoding_verification_row_amd as sv

from _parity import BAND_LOGITS, boundary_mask, check_logits, check_sampled
from _forms import FORMS, set_form

pytestmark = pytest.mark.gpu
DEV = "cuda"
SHAPES = [(16, 5, 9000), (8, 3, 40001), (4, 17, 4100), (6, 1, 130), (24, 5, 128256)]
VARIANTS = ("out_of_range_low", "out_of_range_high", "zero_mass_token", "scaled_copy")


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


def _dev(*arrays):
    return [torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in arrays]


def _planted(B, K, V, seed, logits=False):
    """Workload-c3 rows; every even sequence s gets a zero-residual rejection
    at n = (s // 2) % K.  Returns p, q, t, u (logits when logits=True: the
    log of the rows, -1e4 for zeros), the planted mask and n."""
    rng = np.random.default_rng(seed)
    b = workloads.make_batch("c3", B, K, V, seed=seed)
    p, q = b.target_probs.copy(), b.draft_probs.copy()
    t, u = b.draft_tokens.copy(), b.uniforms.copy()
    planted = np.zeros(B, bool)
    nsel = np.full(B, -1)
    for s in range(0, B, 2):
        n = (s // 2) % K
        variant = VARIANTS[(s // 2) % (3 if logits else 4)]
        for i in range(n):                             # accepted with certainty
            q[s, i] = p[s, i]
            t[s, i] = int(rng.choice(np.flatnonzero(p[s, i] > 0)))
        if variant == "zero_mass_token":
            j = int(rng.integers(0, V))
            p[s, n, j] = 0.0
            t[s, n] = j
        elif variant == "out_of_range_low":
            t[s, n] = -1 - int(rng.integers(0, 1000))
        else:
            t[s, n] = V + int(rng.integers(0, 1000))
        q[s, n] = p[s, n] * np.float32(2.0) if variant == "scaled_copy" else p[s, n]
        planted[s] = True
        nsel[s] = n
    if logits:
        p = np.where(p > 0, np.log(np.maximum(p, 1e-30)), -1e4).astype(np.float32)
        q = np.where(q > 0, np.log(np.maximum(q, 1e-30)), -1e4).astype(np.float32)
    return p, q, t, u, planted, nsel


def _assert_planted(o, planted, nsel):
    assert np.all(o["diag"]["draw_kind"][planted] == 3)
    assert np.array_equal(o["n_accepted"][planted], nsel[planted])


def _fresh_ws(B, K, V):
    ws = torch.empty(sv.sv_workspace_size(B, K, V, True), dtype=torch.uint8, device=DEV)
    sv.sv_workspace_init(ws)
    return ws


def _np(*ts):
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in ts]


# ------------------------------------------------------------- R8 --

@pytest.mark.parametrize("B,K,V", SHAPES, ids=lambda x: str(x))
def test_zero_residual_fallback_probabilities(B, K, V, form):
    _case(f"R8 probabilities B={B} K={K} V={V} form={form}")
    p, q, t, u, planted, nsel = _planted(B, K, V, seed=B * 7 + K * 3 + V)
    o = oracle.verify_sample(p, q, t, u)
    _assert_planted(o, planted, nsel)
    args = _dev(p, q, t, u)
    n, nx, st = sv.sv_verify_sample_batched(*args, stats=True, workspace=_fresh_ws(B, K, V))
    n, nx = _np(n, nx)
    rep = check_sampled(n, nx, sv.stats_to_numpy(st), o)
    n0, nx0 = _np(*sv.sv_verify_sample_batched(*args, workspace=_fresh_ws(B, K, V)))
    ne, nxe = _np(*sv.sv_verify_sample_early_batched(*args, workspace=_fresh_ws(B, K, V)))
    for a, b_ in ((n0, n), (nx0, nx), (ne, n), (nxe, nx)):
        assert np.array_equal(a, b_)
    # the planted sequences are compared, not exempted
    assert not boundary_mask(o["diag"], 1e-9)[planted].any()
    print(f"  parity {rep}")


@pytest.mark.parametrize("B,K,V", SHAPES[:4], ids=lambda x: str(x))
def test_zero_residual_fallback_logits(B, K, V, form):
    _case(f"R8 logits B={B} K={K} V={V} form={form}")
    p, q, t, u, planted, nsel = _planted(B, K, V, seed=B * 11 + K * 5 + V, logits=True)
    tau = 0.9
    o = verify_sample_logits(p, q, t, u, tau)
    _assert_planted(o, planted, nsel)
    args = _dev(p, q, t, u)
    n, nx = _np(*sv.sv_verify_sample_logits_batched(*args[:4], tau, workspace=_fresh_ws(B, K, V)))
    ne, nxe = _np(*sv.sv_verify_sample_logits_early_batched(*args[:4], tau, workspace=_fresh_ws(B, K, V)))
    assert np.array_equal(ne, n) and np.array_equal(nxe, nx)
    rep = check_logits(n, nx, o)
    # n is decided exactly on the planted sequences (no acceptance test is
    # near its ratio: the ratios there are 1 or the token has no weight)
    assert np.array_equal(n[planted], nsel[planted])
    assert (~boundary_mask(o["diag"], BAND_LOGITS))[planted].sum() >= planted.sum() * 3 // 4
    print(f"  parity {rep}")


# ----------------------------------------------------- lost decisions --

@pytest.mark.parametrize("B,K,V", SHAPES, ids=lambda x: str(x))
def test_lost_decisions_probabilities(B, K, V, form, monkeypatch):
    _case(f"lost decisions, probabilities B={B} K={K} V={V} form={form}")
    rng = np.random.default_rng(B + K + V)
    b = workloads.make_batch("c3", B, K, V, seed=int(rng.integers(1 << 20)))
    p, q, t, u = b.target_probs, b.draft_probs, b.draft_tokens, b.uniforms
    o = oracle.verify_sample(p, q, t, u)
    args = _dev(p, q, t, u)
    calls = {
        "full": lambda ws: sv.sv_verify_sample_batched(*args, workspace=ws),
        "stats": lambda ws: sv.sv_verify_sample_batched(*args, stats=True, workspace=ws)[:2],
        "early": lambda ws: sv.sv_verify_sample_early_batched(*args, workspace=ws),
    }
    ref = {k: _np(*f(_fresh_ws(B, K, V))) for k, f in calls.items()}
    monkeypatch.setenv("SV_VERIFY_FORCE_LOST", "1")
    for k, f in calls.items():
        n, nx = _np(*f(_fresh_ws(B, K, V)))
        assert np.array_equal(n, ref[k][0]) and np.array_equal(nx, ref[k][1]), k
        assert np.array_equal(n, ref["full"][0]) and np.array_equal(nx, ref["full"][1]), k
        check_sampled(n, nx, None, o)


@pytest.mark.parametrize("B,K,V", SHAPES, ids=lambda x: str(x))
def test_lost_decisions_logits(B, K, V, form, monkeypatch):
    _case(f"lost decisions, logits B={B} K={K} V={V} form={form}")
    rng = np.random.default_rng(3 * B + K + V)
    b = workloads.make_batch("c3", B, K, V, seed=int(rng.integers(1 << 20)), logits=True)
    tl, dl, t, u = b.target_probs, b.draft_probs, b.draft_tokens, b.uniforms
    tau = 1.1
    o = verify_sample_logits(tl, dl, t, u, tau)
    args = _dev(tl, dl, t, u)
    calls = {
        "full": lambda ws: sv.sv_verify_sample_logits_batched(*args, tau, workspace=ws),
        "early": lambda ws: sv.sv_verify_sample_logits_early_batched(*args, tau, workspace=ws),
    }
    ref = {k: _np(*f(_fresh_ws(B, K, V))) for k, f in calls.items()}
    monkeypatch.setenv("SV_VERIFY_FORCE_LOST", "1")
    for k, f in calls.items():
        n, nx = _np(*f(_fresh_ws(B, K, V)))
        assert np.array_equal(n, ref[k][0]) and np.array_equal(nx, ref[k][1]), k
        assert np.array_equal(n, ref["full"][0]) and np.array_equal(nx, ref["full"][1]), k
        check_logits(n, nx, o)
