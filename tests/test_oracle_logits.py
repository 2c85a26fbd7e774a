"""Pins of the logits oracle (oracle/logits.py): sampled verification on
logits warped by a temperature, softmax(l / tau) being the warped
distribution (a reading; the spec-verify kernel card, section "Method",
requires only that target and draft be warped identically).

1. Exact enumeration at tiny V (as for the probability oracle): every draft
   combination and every cell of the uniforms, weighted exactly; the cells'
   outcomes and the emitted-token law prod_{i<j} alpha_i * p_hat_j, with
   p_hat = scipy's softmax of l / tau (an independent definition), within
   1e-12.
2. Agreement with the probability oracle (sv_oracle.c) on the f32-rounded
   softmax of the same logits: identical outputs on every sequence that is
   not within 1e-5 of a decision boundary on either side.
3. Exact invariances of the warp: adding a constant to a row of logits, and
   scaling logits and temperature together, change nothing, bit for bit.
4. The low-temperature limit: with a greedy draft (each draft token its
   row's argmax), integer logits whose maximum is unique, tau = 1/64 and
   uniforms in [1e-6, 1), the outputs are those of greedy verification of
   the target (the greedy oracle, sv_oracle.c), exactly.
"""
import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
from oracle.logits import verify_sample_logits, warp_row

from test_oracle_law import _cells
from _parity import boundary_mask


def _logit_instance(rng, K, V, zeros=True):
    """Small integer logits (exact in f32); some entries -1e4, whose weight
    underflows to exactly 0 at the temperatures used."""
    def row():
        z = rng.integers(-3, 4, size=V).astype(np.float32)
        if zeros and V > 2:
            z[rng.choice(V, size=rng.integers(0, V // 2), replace=False)] = -1e4
        return z
    return np.stack([row() for _ in range(K + 1)]), (np.stack([row() for _ in range(K)]) if K else
                                                    np.zeros((0, V), np.float32))


@pytest.mark.parametrize("K,V,tau,seed", [(0, 2, 1.0, 0), (0, 8, 0.5, 1), (1, 3, 2.0, 2), (1, 6, 0.75, 3),
                                          (2, 4, 1.0, 4), (2, 6, 1.5, 5), (3, 5, 0.5, 6), (3, 8, 1.0, 7)])
def test_logits_enumeration_preserves_warped_law(K, V, tau, seed):
    rng = np.random.default_rng(2000 + seed)
    lp, lq = _logit_instance(rng, K, V)
    tau32 = float(np.float32(tau))
    ph = softmax(lp.astype(np.float64) / tau32, axis=1)
    qh = softmax(lq.astype(np.float64) / tau32, axis=1) if K else np.zeros((0, V))
    t, u, wts, expect = _cells(ph, qh)
    B = len(wts)
    r = verify_sample_logits(np.broadcast_to(lp, (B, K + 1, V)), np.broadcast_to(lq, (B, K, V)), t, u, tau)
    got = list(zip(r["n_accepted"].tolist(), r["next_token"].tolist()))
    assert got == expect
    emit = np.zeros((K + 1, V))
    for c in range(B):
        n, nxt = got[c]
        for j, x in enumerate(list(t[c, :n]) + [nxt]):
            emit[j, x] += wts[c]
    alpha = [np.minimum(ph[i], qh[i]).sum() for i in range(K)]
    reach = 1.0
    for j in range(K + 1):
        np.testing.assert_allclose(emit[j], reach * ph[j], rtol=0, atol=1e-12)
        if j < K:
            reach *= alpha[j]


def _boundary(d):
    return boundary_mask(d, 1e-5)


@pytest.mark.parametrize("tau", [0.6, 1.0, 1.7])
def test_logits_agree_with_probability_oracle(tau):
    rng = np.random.default_rng(int(tau * 100))
    B, K, V = 96, 4, 3000
    lp = rng.normal(0, 2.0, (B, K + 1, V)).astype(np.float32)
    lq = (lp[:, :K] + rng.normal(0, 1.0, (B, K, V))).astype(np.float32)
    tau32 = float(np.float32(tau))
    qh = softmax(lq.astype(np.float64) / tau32, axis=2)
    t = np.array([[rng.choice(V, p=qh[b, i]) for i in range(K)] for b in range(B)], np.int32)
    u = rng.random((B, K + 1), dtype=np.float32)
    rl = verify_sample_logits(lp, lq, t, u, tau)
    p32 = softmax(lp.astype(np.float64) / tau32, axis=2).astype(np.float32)
    q32 = qh.astype(np.float32)
    rp = oracle.verify_sample(p32, q32, t, u)
    ok = ~(_boundary(rl["diag"]) | _boundary(rp["diag"]))
    assert ok.sum() >= B * 3 // 4   # the 1e-5 band covers ~V * 2e-5 of the final draws
    assert np.array_equal(rl["n_accepted"][ok], rp["n_accepted"][ok])
    assert np.array_equal(rl["next_token"][ok], rp["next_token"][ok])
    # each row's mass is exp(logsumexp(l / tau) - max l / tau) (scipy, independently)
    lse = logsumexp(lp.astype(np.float64) / tau32, axis=2) - lp.max(axis=2).astype(np.float64) / tau32
    np.testing.assert_allclose(rl["P"], np.exp(lse), rtol=1e-12)
    assert np.all(rl["n_accepted"] <= K) and np.all((rl["next_token"] >= 0) & (rl["next_token"] < V))


def test_warp_invariances_are_exact():
    rng = np.random.default_rng(5)
    B, K, V = 40, 3, 500
    lp = rng.integers(-20, 21, (B, K + 1, V)).astype(np.float32)
    lq = rng.integers(-20, 21, (B, K, V)).astype(np.float32)
    t = rng.integers(0, V, (B, K)).astype(np.int32)
    t[:, 0] = np.argmax(lq[:, 0], axis=1)   # some acceptances
    u = rng.random((B, K + 1), dtype=np.float32)
    base = verify_sample_logits(lp, lq, t, u, 0.75)
    shifted = verify_sample_logits(lp + np.float32(7), lq - np.float32(3), t, u, 0.75)
    scaled = verify_sample_logits(lp * np.float32(2), lq * np.float32(2), t, u, 1.5)
    for r in (shifted, scaled):
        assert np.array_equal(r["n_accepted"], base["n_accepted"])
        assert np.array_equal(r["next_token"], base["next_token"])
        assert r["P"].tobytes() == base["P"].tobytes() and r["Q"].tobytes() == base["Q"].tobytes()
    assert 0 < base["n_accepted"].mean() < K
    # the warp itself: the maximum has weight exactly 1
    w = warp_row(lp[0, 0], 0.75)
    assert w.max() == 1.0 and np.all(w > 0)


def test_logits_preconditions():
    lp = np.zeros((1, 2, 4), np.float32)
    lq = np.zeros((1, 1, 4), np.float32)
    t = np.zeros((1, 1), np.int32)
    u = np.zeros((1, 2), np.float32)
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(oracle.OracleError):
            verify_sample_logits(lp, lq, t, u, bad)
    lp2 = lp.copy()
    lp2[0, 0, 1] = np.inf
    with pytest.raises(oracle.OracleError):
        verify_sample_logits(lp2, lq, t, u, 1.0)
    # all-equal logits: uniform rows, the draft token is accepted (rho = 1 > u)
    r = verify_sample_logits(lp, lq, t, u, 1.0)
    assert r["n_accepted"][0] == 1 and r["next_token"][0] == 0


def greedy_limit_instance(rng, B, K, V):
    """Integer logits in [-20, 20] with one maximum per row, raised 1 above
    the rest; draft tokens the argmax of their draft row, each row's draft
    argmax placed at the target's argmax about half the time."""
    def rows(n):
        z = rng.integers(-20, 21, size=(B, n, V)).astype(np.float32)
        top = rng.integers(0, V, size=(B, n))
        return z, top
    lp, tp_top = rows(K + 1)
    lq, tq_top = rows(K)
    same = rng.random((B, K)) < 0.5
    tq_top = np.where(same, tp_top[:, :K], tq_top)
    for z, top in ((lp, tp_top), (lq, tq_top)):
        bi, ri = np.meshgrid(np.arange(B), np.arange(z.shape[1]), indexing="ij")
        z[bi, ri, top] = z.max(axis=2) + 1
    t = tq_top.astype(np.int32)
    u = rng.uniform(1e-6, 1.0, (B, K + 1)).astype(np.float32)
    return lp, lq, t, u


def test_low_temperature_limit_is_greedy_verification():
    """At tau = 1/64 every weight but a row's maximum is at most e^-64
    (logit gap >= 1).  A draft token at the target's argmax has
    p(t) >= 1 - V e^-64 >= q(t) - V e^-64 and is accepted (u < 1 - 2^-24);
    one elsewhere has p(t) / q(t) <= e^-64 / (1 - V e^-64) < u and is
    rejected; the residual and the bonus row put all but V e^-64 of their
    mass on the target's argmax, which every u in [1e-6, 1 - 2^-24] lands on.
    So the outputs are greedy verification's, whatever the seed."""
    rng = np.random.default_rng(64)
    B, K, V = 300, 4, 700
    lp, lq, t, u = greedy_limit_instance(rng, B, K, V)
    r = verify_sample_logits(lp, lq, t, u, 1.0 / 64)
    w = np.exp(lp.astype(np.float64) - lp.max(axis=2, keepdims=True)).astype(np.float32)
    g = oracle.verify_greedy(w, t)
    assert np.array_equal(r["n_accepted"], g["n_accepted"])
    assert np.array_equal(r["next_token"], g["next_token"])
    # every outcome occurs
    assert set(np.unique(g["n_accepted"])) == set(range(K + 1))


def test_logits_zero_residual_draws_from_target_row():
    """R8 on logits: draft logits equal to the target's bit for bit give
    identical weights and masses, so a rejected token (out of range here)
    leaves a residual of exactly 0 and the draw is inverse-CDF sampling of
    the warped target row n with u_K; the expected token comes from scipy's
    softmax of l / tau (outside a 1e-9 band around the CDF's breakpoints)."""
    rng = np.random.default_rng(808)
    B, K, V, tau = 40, 4, 700, 0.8
    lp = rng.normal(0, 2.0, (B, K + 1, V)).astype(np.float32)
    lq = (lp[:, :K] + rng.normal(0, 1.0, (B, K, V))).astype(np.float32)
    t = rng.integers(0, V, size=(B, K)).astype(np.int32)
    u = rng.random((B, K + 1), dtype=np.float32)
    nsel = rng.integers(0, K, size=B)
    for b in range(B):
        n = int(nsel[b])
        lq[b, :n + 1] = lp[b, :n + 1]                 # rows 0..n: identical warps
        t[b, :n] = np.argmax(lp[b, :n], axis=1)       # accepted with certainty
        t[b, n] = V if b % 2 else -1                  # rejected
    r = verify_sample_logits(lp, lq, t, u, tau)
    tau32 = float(np.float32(tau))
    checked = 0
    for b in range(B):
        n = int(nsel[b])
        assert int(r["n_accepted"][b]) == n
        assert int(r["diag"]["draw_kind"][b]) == 3
        c = np.cumsum(softmax(lp[b, n].astype(np.float64) / tau32))
        T = float(u[b, K]) * c[-1]
        if np.min(np.abs(c - T)) <= 1e-9 * c[-1]:
            continue
        assert int(r["next_token"][b]) == int(np.searchsorted(c, T, side="right"))
        checked += 1
    assert checked >= B - 2


def test_logits_rounding_guard_hand_derived():
    """The guard's one reachable case, derived by hand.  V = 2, K = 1,
    tau = 1.  Target row 0 has logits (0, -744.4): weights 1 and
    exp(-744.4), which rounds to the smallest fp64 subnormal 2^-1074; its
    mass 1 + 2^-1074 rounds to 1.  Draft row 0 has logits (0, -2000):
    weights 1 and 0, mass 1.  The token 2 is outside [0, 2), so it is
    rejected, and the residual max(0, w_p Q - w_q P) is (0, 2^-1074):
    W = 2^-1074.  With u_1 = 0.75, T = 0.75 * 2^-1074 rounds to 2^-1074 = W,
    no running sum exceeds T, and the guard takes the last position with
    weight, 1 (draw kind 1 + 4).  With u_1 = 0.25, T rounds to 0 and the
    running sum 2^-1074 at position 1 exceeds it: the ordinary rule gives
    position 1 (kind 1) with a draw margin of 0 (T equals C(0) = 0)."""
    lp = np.array([[[0.0, -744.4], [0.0, 0.0]]], np.float32)
    lq = np.array([[[0.0, -2000.0]]], np.float32)
    t = np.array([[2]], np.int32)
    r = verify_sample_logits(lp, lq, t, np.array([[0.5, 0.75]], np.float32), 1.0)
    d = r["diag"][0]
    assert (int(r["n_accepted"][0]), int(r["next_token"][0])) == (0, 1)
    assert int(d["draw_kind"]) == 5 and d["W"] == 2.0 ** -1074 and d["T"] == 2.0 ** -1074
    r = verify_sample_logits(lp, lq, t, np.array([[0.5, 0.25]], np.float32), 1.0)
    d = r["diag"][0]
    assert (int(r["next_token"][0]), int(d["draw_kind"])) == (1, 1)
    assert d["T"] == 0.0 and d["draw_margin"] == 0.0
