"""Distribution-level pins of the sampled oracle.

1. Exact enumeration at tiny V: every draft-token combination and every cell
   of the uniforms is visited once, weighted by its exact probability, so the
   law of the emitted tokens is computed exactly (up to fp64 rounding).
   Speculative sampling preserves the target law (the spec-verify kernel
   card, section "Method", sampling bullet, and "Correctness"): the token at
   position j is emitted with probability prod_{i<j} alpha_i * p_hat_j(x),
   alpha_i = sum_x min(p_hat_i, q_hat_i).  Checked within 1e-12.
2. The analytic accepted-length law ("Measured" and "Correctness"): over
   seeded rounds the mean of n_accepted matches sum_{i=1..K} prod_{j<i}
   alpha_j (the card's sum_i alpha^i when the alpha_j are equal) within three
   standard errors.
"""
import itertools

import numpy as np
import pytest

import workloads


def _instance(rng, K, V, zeros=True, ties=True):
    """Integer masses 0..16 (some zero), random scales: every cell of the
    enumeration is at least ~1e-4 wide, so its f32 midpoint is interior."""
    def row():
        m = rng.integers(1, 17, size=V).astype(np.float64)
        if zeros and V > 2:
            m[rng.choice(V, size=rng.integers(0, V // 2), replace=False)] = 0.0
        if ties and V > 2 and rng.random() < 0.5:
            m[rng.choice(V, size=2, replace=False)] = m.max()
        if m.sum() == 0:
            m[0] = 1.0
        return m
    scale_p = rng.choice([0.25, 0.5, 1.0, 2.0, 4.0], size=K + 1)
    scale_q = rng.choice([0.25, 0.5, 1.0, 2.0, 4.0], size=K)
    p = np.stack([row() * s / 16.0 for s in scale_p]).astype(np.float32)
    q = np.stack([row() * s / 16.0 for s in scale_q]).astype(np.float32) if K else np.zeros((0, V), np.float32)
    return p, q


def _cells(p, q):
    """All (t, u) cells with their exact weights and the outcome they define."""
    K1, V = p.shape
    K = K1 - 1
    P = p.astype(np.float64).sum(axis=1)
    Q = q.astype(np.float64).sum(axis=1)
    ph = p.astype(np.float64) / P[:, None]
    qh = q.astype(np.float64) / Q[:, None] if K else q
    rows_t, rows_u, weights, expect = [], [], [], []
    for t in itertools.product(range(V), repeat=K):
        wt = 1.0
        for i in range(K):
            wt *= qh[i, t[i]]
        if wt == 0.0:
            continue
        a = [min(1.0, ph[i, t[i]] / qh[i, t[i]]) for i in range(K)]
        for n in range(K + 1):
            wpath = wt
            u = np.zeros(K + 1)
            for i in range(n):
                wpath *= a[i]
                u[i] = 0.5 * a[i]
            if n < K:
                wpath *= 1.0 - a[n]
                u[n] = 0.5 * (1.0 + a[n])
                r = np.maximum(ph[n] - qh[n], 0.0)
            else:
                r = ph[K].copy()
            if wpath == 0.0:
                continue
            c = np.cumsum(r) / r.sum()
            lo = 0.0
            for x in range(V):
                hi = c[x]
                if hi > lo:
                    u[K] = 0.5 * (lo + hi)
                    u32 = u.astype(np.float32)
                    # the f32 midpoints stay strictly inside their cells
                    for i in range(n):
                        assert u32[i] < a[i]
                    if n < K:
                        assert u32[n] >= a[n]
                    assert lo < u32[K] < hi
                    rows_t.append(t)
                    rows_u.append(u32)
                    weights.append(wpath * (hi - lo))
                    expect.append((n, x))
                lo = hi
    return (np.array(rows_t, np.int32).reshape(len(weights), K), np.array(rows_u, np.float32),
            np.array(weights), expect)


@pytest.mark.parametrize("K,V,seed", [(0, 2, 0), (0, 8, 1), (1, 2, 2), (1, 5, 3), (1, 8, 4),
                                      (2, 3, 5), (2, 6, 6), (3, 4, 7), (3, 8, 8)])
def test_exact_enumeration_preserves_target_law(oracle_mod, K, V, seed):
    rng = np.random.default_rng(1000 + seed)
    p, q = _instance(rng, K, V)
    t, u, wts, expect = _cells(p, q)
    B = len(wts)
    tp = np.broadcast_to(p, (B, K + 1, V)).copy()
    dp = np.broadcast_to(q, (B, K, V)).copy()
    r = oracle_mod.verify_sample(tp, dp, t, u)
    # every cell midpoint maps to the cell's outcome
    got = list(zip(r["n_accepted"].tolist(), r["next_token"].tolist()))
    assert got == expect
    # law of the emitted tokens, from the oracle's outputs
    emit = np.zeros((K + 1, V))
    for c in range(B):
        n, nxt = got[c]
        seq = list(t[c, :n]) + [nxt]
        for j, x in enumerate(seq):
            emit[j, x] += wts[c]
    P = p.astype(np.float64).sum(axis=1)
    ph = p.astype(np.float64) / P[:, None]
    alpha = [np.minimum(ph[i], q[i].astype(np.float64) / q[i].astype(np.float64).sum()).sum()
             for i in range(K)]
    reach = 1.0
    for j in range(K + 1):
        np.testing.assert_allclose(emit[j], reach * ph[j], rtol=0, atol=1e-12)
        if j < K:
            reach *= alpha[j]
    assert abs(wts.sum() - 1.0) < 1e-12


def _law_check(oracle_mod, batches):
    ns, means, vars_ = [], [], []
    for b in batches:
        r = oracle_mod.verify_sample(b.target_probs, b.draft_probs, b.draft_tokens, b.uniforms)
        for s in range(b.target_probs.shape[0]):
            m, v = oracle_mod.expected_accepted_length(r["alpha"][s])
            ns.append(int(r["n_accepted"][s]))
            means.append(m)
            vars_.append(v)
    ns, means, vars_ = np.array(ns), np.array(means), np.array(vars_)
    se = np.sqrt(vars_.sum()) / len(ns)
    return ns.mean(), means.mean(), se


def test_accepted_length_law_config1_600_rounds(oracle_mod):
    """Workload 1 (B=1, K=4, V=32000), 600 seeded rounds, as on the card's
    'Measured' section: empirical mean of n within 3 SE of the analytic law."""
    batches = [workloads.make_config(1, rnd=r) for r in range(600)]
    emp, ana, se = _law_check(oracle_mod, batches)
    assert abs(emp - ana) <= 3 * se, (emp, ana, se)
    # the workload's acceptance is the calibrated 0.68
    alphas = np.concatenate([oracle_mod.verify_sample(b.target_probs, b.draft_probs, b.draft_tokens,
                                                      b.uniforms)["alpha"].ravel() for b in batches[:20]])
    assert abs(alphas.mean() - 0.68) < 0.01


@pytest.mark.parametrize("family,B,K,V", [("c3", 512, 5, 4096), ("c4", 512, 8, 4096), ("c5", 256, 16, 8192)])
def test_accepted_length_law_heterogeneous(oracle_mod, family, B, K, V):
    b = workloads.make_batch(family, B, K, V, seed=3)
    emp, ana, se = _law_check(oracle_mod, [b])
    assert abs(emp - ana) <= 3 * se, (emp, ana, se)


def test_config4_q_equals_p_quarter_accepts_all(oracle_mod):
    b = workloads.make_batch("c4", 64, 8, 2048, seed=4)
    r = oracle_mod.verify_sample(b.target_probs, b.draft_probs, b.draft_tokens, b.uniforms)
    qeqp = np.array([s["q_equals_p"] for s in b.info["per_seq"]])
    assert qeqp.sum() == 16
    assert np.all(r["n_accepted"][qeqp] == 8)
    assert np.all(r["alpha"][qeqp] == pytest.approx(1.0, abs=1e-12))
