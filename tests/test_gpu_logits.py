"""GPU parity of the logits entry point (sv_verify_sample_logits_batched)
against the fp64 logits oracle (oracle/logits.py), through the C ABI.

The bar is that of the sampled path: n_accepted and next_token identical on
every sequence whose decisions all lie more than 1e-5 of their mass from a
boundary (the oracle's margins); boundary sequences are counted.  The kernel
warps each value in fp32 (exp2 of an fp32 argument), so its weights near a
row's maximum differ from the oracle's fp64 exp by ~1e-7 relative: far
inside that band.  An acceptance test's two weights, whose exponents can be
far below fp32's range at a low temperature, are taken with fp64 range
(the extreme-temperature and low-temperature-limit cases reach that path).
"""
import os

import numpy as np
import pytest
import torch

from oracle.logits import verify_sample_logits
import workloads
from workloads.device import device_batch
import speculative_decoding_verification_row_amd as sv

from _parity import BAND_LOGITS, boundary_mask, check_logits

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


# Both forms of the pass (walks down the draft rows, one block per draft
# row); SV_VERIFY_ROWS forces one, the library otherwise picks by size.
@pytest.fixture(params=["walks", "rows"])
def form(request, monkeypatch):
    monkeypatch.setenv("SV_VERIFY_ROWS", "1" if request.param == "rows" else "0")
    return request.param


def _boundary(d):
    return boundary_mask(d, BAND_LOGITS)


check = check_logits


def run(tl, dl, t, u, tau, offset=False, **kw):
    """The library on host arrays; offset=True places the rows at a 4- but
    not 16-byte aligned address (the scalar load path)."""
    B, K1, V = tl.shape
    K = K1 - 1
    if offset:
        bp = torch.zeros(tl.size + 1, dtype=torch.float32, device=DEV)
        bq = torch.zeros(dl.size + 1, dtype=torch.float32, device=DEV)
        tld, dld = bp[1:].view(B, K1, V), bq[1:].view(B, K, V)
        tld.copy_(torch.from_numpy(np.ascontiguousarray(tl)))
        dld.copy_(torch.from_numpy(np.ascontiguousarray(dl)))
    else:
        tld = torch.from_numpy(np.ascontiguousarray(tl)).to(DEV)
        dld = torch.from_numpy(np.ascontiguousarray(dl)).to(DEV)
    n, nx = sv.sv_verify_sample_logits_batched(tld, dld, torch.from_numpy(t).to(DEV),
                                               torch.from_numpy(u).to(DEV), tau, **kw)
    torch.cuda.synchronize()
    return n.cpu().numpy(), nx.cpu().numpy()


def _rows(rng, B, K, V, tau):
    """Logits N(0, 2^2), draft = target + N(0, 1); some entries at -1e4
    (weight 0), some rows with a tied maximum; tokens drawn from the warped
    draft, a few random and a few outside [0, V)."""
    lp = rng.normal(0.0, 2.0, (B, K + 1, V)).astype(np.float32)
    lq = (lp[:, :K] + rng.normal(0.0, 1.0, (B, K, V))).astype(np.float32)
    if V > 4:
        lp[rng.random(lp.shape) < 0.1] = -1e4
        lq[rng.random(lq.shape) < 0.1] = -1e4
        for b in range(B):
            i = rng.integers(0, K + 1)
            lp[b, i, rng.choice(V, 2, replace=False)] = lp[b, i].max()
    t = np.zeros((B, K), np.int32)
    for b in range(B):
        for i in range(K):
            r = rng.random()
            if r < 0.05:
                t[b, i] = V + int(rng.integers(0, 3))
            elif r < 0.2:
                t[b, i] = rng.integers(0, V)
            else:
                z = lq[b, i].astype(np.float64) / tau
                w = np.exp(z - z.max())
                t[b, i] = min(int(np.searchsorted(np.cumsum(w), rng.random() * w.sum(), side="right")), V - 1)
    u = rng.random((B, K + 1), dtype=np.float32)
    return lp, lq, t, u


SMALL = [(1, 0, 1), (3, 0, 7), (2, 1, 2), (4, 2, 3), (5, 4, 1000), (3, 3, 1003), (2, 2, 4096),
         (2, 3, 4097), (2, 2, 16389), (3, 4, 32000), (2, 5, 40001), (1, 2, 65540), (2, 130, 5000)]


@pytest.mark.parametrize("tau", [0.5, 1.0, 2.0])
@pytest.mark.parametrize("B,K,V", SMALL, ids=lambda x: str(x))
def test_logits_small(B, K, V, tau, form):
    _case(f"logits small B={B} K={K} V={V} tau={tau} form={form}")
    rng = np.random.default_rng(B * 1000 + K * 100 + V + int(tau * 10))
    lp, lq, t, u = _rows(rng, B, K, V, tau)
    o = verify_sample_logits(lp, lq, t, u, tau)
    check(*run(lp, lq, t, u, tau), o)
    check(*run(lp, lq, t, u, tau, offset=True), o)


def test_logits_max_vocabulary(form):
    """V = 524288: 128 chunks per row (wave 0's lanes hold two chunks each)."""
    _case(f"logits V=524288 B=2 K=3 form={form}")
    rng = np.random.default_rng(99)
    lp, lq, t, u = _rows(rng, 2, 3, 524288, 1.0)
    check(*run(lp, lq, t, u, 1.0), verify_sample_logits(lp, lq, t, u, 1.0))


def _slow_path_flag(ws):
    return int(ws[4:8].cpu().numpy().view(np.uint32)[0])


@pytest.mark.parametrize("tau", [1.0, 0.6])
def test_logits_full_size(tau):
    B, K, V = 256, 5, 128256
    _case(f"logits full size B={B} K={K} V={V} tau={tau} (generating)")
    db = device_batch("c3", B, K, V, seed=0, device=DEV, logits=True)
    ws = sv.workspace_for(B, K, V, True, DEV)
    sv.sv_workspace_init(ws)   # only this call can set the recompute flag
    _case("logits full size: running")
    n, nx = sv.sv_verify_sample_logits_batched(db["tp"], db["dp"], db["dt"], db["u"], tau, workspace=ws)
    torch.cuda.synchronize()
    n, nx = n.cpu().numpy(), nx.cpu().numpy()
    assert _slow_path_flag(ws) == 0
    rows = None if tau == 1.0 else np.arange(0, B, 4)
    hb = workloads.make_batch("c3", B, K, V, seed=0, seqs=rows, logits=True)
    o = verify_sample_logits(hb.target_probs, hb.draft_probs, hb.draft_tokens, hb.uniforms, tau)
    sel = slice(None) if rows is None else rows
    rep = check(n[sel], nx[sel], o)
    print(f"  parity {rep}")
    assert 0 < n.mean() < K


def test_logits_recompute_path_is_bit_identical(form, monkeypatch):
    _case(f"logits forced recompute B=6 K=5 V=40000 form={form}")
    rng = np.random.default_rng(7)
    lp, lq, t, u = _rows(rng, 6, 5, 40000, 0.8)
    ref = run(lp, lq, t, u, 0.8)
    ws = torch.empty(sv.sv_workspace_size(6, 5, 40000, True), dtype=torch.uint8, device=DEV)
    sv.sv_workspace_init(ws)
    monkeypatch.setenv("SV_VERIFY_FORCE_RECOMPUTE", "1")
    got = run(lp, lq, t, u, 0.8, workspace=ws)
    monkeypatch.delenv("SV_VERIFY_FORCE_RECOMPUTE")
    torch.cuda.synchronize()
    assert _slow_path_flag(ws) == 1
    assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])
    check(*got, verify_sample_logits(lp, lq, t, u, 0.8))


def test_logits_agree_with_probability_kernel():
    """The probability entry point on the f32-rounded softmax of the same
    logits: both agree with their oracles, so outside the boundary band of
    either they agree with each other."""
    _case("logits vs probability kernel B=32 K=4 V=50000 tau=0.9")
    rng = np.random.default_rng(11)
    B, K, V, tau = 32, 4, 50000, 0.9
    lp, lq, t, u = _rows(rng, B, K, V, tau)
    tau32 = float(np.float32(tau))

    def sm(z):
        z = z.astype(np.float64) / tau32
        e = np.exp(z - z.max(axis=-1, keepdims=True))
        return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)
    n_l, x_l = run(lp, lq, t, u, tau)
    p = torch.from_numpy(sm(lp)).to(DEV)
    q = torch.from_numpy(sm(lq)).to(DEV)
    n_p, x_p = sv.sv_verify_sample_batched(p, q, torch.from_numpy(t).to(DEV), torch.from_numpy(u).to(DEV))
    n_p, x_p = n_p.cpu().numpy(), x_p.cpu().numpy()
    o = verify_sample_logits(lp, lq, t, u, tau)
    ok = ~_boundary(o["diag"])
    assert ok.sum() >= B // 2
    assert np.array_equal(n_l[ok], n_p[ok]) and np.array_equal(x_l[ok], x_p[ok])


def test_logits_argument_errors():
    _case("logits argument errors")
    tl = torch.zeros((1, 2, 8), dtype=torch.float32, device=DEV)
    dl = torch.zeros((1, 1, 8), dtype=torch.float32, device=DEV)
    t = torch.zeros((1, 1), dtype=torch.int32, device=DEV)
    u = torch.zeros((1, 2), dtype=torch.float32, device=DEV)
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(sv.SVError):
            sv.sv_verify_sample_logits_batched(tl, dl, t, u, bad)
    n, nx = sv.sv_verify_sample_logits_batched(tl, dl, t, u, 1.0)
    assert int(n.item()) == 1 and int(nx.item()) == 0


@pytest.mark.parametrize("tau", [0.02, 50.0])
@pytest.mark.parametrize("B,K,V", [(4, 3, 5000), (2, 5, 40001)], ids=lambda x: str(x))
def test_logits_extreme_temperatures(B, K, V, tau, form):
    """A very low temperature (most fp32 weights underflow to 0, where the
    fp64 oracle keeps them, far below the 1e-5 band) and a very high one
    (nearly flat rows)."""
    _case(f"logits extreme tau={tau} B={B} K={K} V={V} form={form}")
    rng = np.random.default_rng(int(tau * 100) + B + K + V)
    lp, lq, t, u = _rows(rng, B, K, V, tau)
    check(*run(lp, lq, t, u, tau), verify_sample_logits(lp, lq, t, u, tau))


@pytest.mark.parametrize("B,K,V", [(300, 4, 700), (8, 5, 40001), (256, 5, 128256)], ids=lambda x: str(x))
def test_logits_low_temperature_is_greedy(B, K, V, form):
    """The low-temperature limit (pinned on the oracle): a greedy draft over
    integer logits with unique row maxima at tau = 1/64 gives exactly the
    outputs of greedy verification of the target, at any size; here up to
    the B=256 K=5 V=128256 shape.  Every rejection's token weight lies
    below e^-64 of its row's, beyond the fp32 fast test, so the fp64 test
    decides those rows."""
    from test_oracle_logits import greedy_limit_instance
    _case(f"logits tau=1/64 greedy limit B={B} K={K} V={V} form={form}")
    lp, lq, t, u = greedy_limit_instance(np.random.default_rng(B + K + V), B, K, V)
    n, nx = run(lp, lq, t, u, 1.0 / 64)
    am = lp.argmax(axis=2)                                   # the unique maximum of each row
    miss = np.concatenate([t != am[:, :K], np.ones((B, 1), bool)], axis=1)
    want_n = miss.argmax(axis=1).astype(np.int32)
    want_x = am[np.arange(B), want_n].astype(np.int32)
    assert np.array_equal(n, want_n)
    assert np.array_equal(nx, want_x)


@pytest.mark.parametrize("B,K,V", [(4, 3, 5000), (2, 5, 40001)], ids=lambda x: str(x))
def test_logits_large_offsets(B, K, V, form):
    """Logits far from 0 (target +1e5, draft -3e4, each row its own extra
    offset) at tau = 0.5: the fp32 rounding of max l * log2(e) / tau is then
    2^-5 or so and scales every weight of a row alike, so it must cancel;
    the outputs equal the oracle's on the same f32 logits."""
    _case(f"logits large offsets B={B} K={K} V={V} form={form}")
    rng = np.random.default_rng(B * 7 + K + V)
    lp, lq, t, u = _rows(rng, B, K, V, 0.5)
    lp = (lp + np.float32(1e5) + rng.uniform(-500, 500, (B, K + 1, 1)).astype(np.float32)).astype(np.float32)
    lq = (lq - np.float32(3e4) + rng.uniform(-500, 500, (B, K, 1)).astype(np.float32)).astype(np.float32)
    check(*run(lp, lq, t, u, 0.5), verify_sample_logits(lp, lq, t, u, 0.5))


def test_logits_underflowing_token_weights(form):
    """Draft tokens whose warped weights both lie far below fp32's range at
    tau = 0.02 (exponents near -650 and -720): row 0 of sequence 0 has the
    token 9 below the target row's maximum and 10 below the draft row's, a
    ratio p(t)/q(t) of 2^72, and must be accepted; sequence 1 mirrors it
    (ratio 2^-72) and must be rejected.  In fp32 both weights would be 0 and
    the test 0 < 0 would reject both."""
    _case(f"logits underflowing token weights tau=0.02 form={form}")
    B, K, V, tau = 2, 2, 5000, 0.02
    rng = np.random.default_rng(77)
    lp = rng.normal(0.0, 2.0, (B, K + 1, V)).astype(np.float32)
    lq = rng.normal(0.0, 2.0, (B, K, V)).astype(np.float32)
    t = np.array([[17, 4001], [17, 4001]], np.int32)
    for b, (gp, gq) in enumerate([(9.0, 10.0), (10.0, 9.0)]):
        lp[b, 0, 17] = lp[b, 0].max() - np.float32(gp)
        lq[b, 0, 17] = lq[b, 0].max() - np.float32(gq)
    u = np.full((B, K + 1), 0.5, np.float32)
    o = verify_sample_logits(lp, lq, t, u, tau)
    assert o["n_accepted"][0] >= 1 and o["n_accepted"][1] == 0
    n, nx = run(lp, lq, t, u, tau)
    check(n, nx, o)
    assert n[0] >= 1 and n[1] == 0
