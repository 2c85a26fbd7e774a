"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself:
hand-derived golden cases, special cases that reduce to a library routine
(numpy.argmax, numpy.searchsorted over a cumulative sum), invariants of the
greedy contract, closed forms of speculative sampling, and correctly rounded
sums (math.fsum).  Sources: the spec-verify kernel card, sections "Method",
"Correctness" and "Requirements and limits".
"""
import json
import math
import os

import numpy as np
import pytest

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "verify_cases.json")


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_golden_hand_derived(oracle_mod, case):
    V, K = case["V"], case["K"]
    p = np.array(case["p"], np.float32).reshape(K + 1, V)
    t = np.array(case["t"], np.int32).reshape(K)
    if case["mode"] == "greedy":
        r = oracle_mod.verify_greedy(p, t)
    else:
        q = np.array(case["q"], np.float32).reshape(K, V)
        u = np.array(case["u"], np.float32).reshape(K + 1)
        r = oracle_mod.verify_sample(p, q, t, u)
    assert int(r["n_accepted"][0]) == case["expect"]["n_accepted"]
    assert int(r["next_token"][0]) == case["expect"]["next_token"]
    if "draw_kind" in case["expect"]:
        d = r["diag"][0]
        assert int(d["draw_kind"]) == case["expect"]["draw_kind"]
        for f in ("accept_margin", "draw_margin"):
            want = _fraction(case["expect"][f])
            got = float(d[f])
            assert (got == want) if math.isinf(want) else abs(got - want) <= 1e-15 * max(1.0, want), (f, got, want)


def _fraction(s: str) -> float:
    """'inf', '0', '1/6' -> float."""
    if s == "inf":
        return math.inf
    num, _, den = s.partition("/")
    return float(num) / float(den or 1)


# ------------------------------------------------------------ greedy (P-a) --

def _tie_batch(B, K, V, seed):
    """Rows with planted exact ties of the maximum (2-4 ways) at random
    positions, plus draft tokens that hit the first, a later tied index, or a
    random token."""
    rng = np.random.default_rng(seed)
    p = rng.random((B, K + 1, V)).astype(np.float32)
    for b in range(B):
        for i in range(K + 1):
            k = int(rng.integers(2, 5))
            idx = rng.choice(V, size=k, replace=False)
            p[b, i, idx] = np.float32(2.0)
    t = np.empty((B, K), np.int32)
    for b in range(B):
        for i in range(K):
            ties = np.flatnonzero(p[b, i] == p[b, i].max())
            r = rng.random()
            t[b, i] = ties[0] if r < 0.6 else (ties[-1] if r < 0.8 else rng.integers(0, V))
    return p, t


@pytest.mark.parametrize("family,B,K,V", [("c1", 16, 4, 1000), ("c2", 64, 4, 2048),
                                          ("c5", 8, 16, 4096), ("c3", 16, 5, 1003)])
def test_greedy_equals_plain_greedy_decoding(oracle_mod, family, B, K, V):
    b = workloads.make_batch(family, B, K, V, seed=11)
    r = oracle_mod.verify_greedy(b.target_probs, b.draft_tokens)
    _check_greedy(r, b.target_probs, b.draft_tokens)


def test_greedy_ties_lowest_index(oracle_mod):
    p, t = _tie_batch(64, 3, 37, seed=5)
    r = oracle_mod.verify_greedy(p, t)
    _check_greedy(r, p, t)


def _check_greedy(r, p, t):
    B, K1, V = p.shape
    K = K1 - 1
    am = np.argmax(p, axis=2)                # first occurrence
    assert np.array_equal(r["stats"]["argmax"], am)
    assert np.array_equal(r["stats"]["max_p"], p.max(axis=2))
    for b in range(B):
        n, nxt = int(r["n_accepted"][b]), int(r["next_token"][b])
        # plain greedy decoding of the rows emits argmax_0, argmax_1, ...;
        # the verifier emits t_0..t_{n-1}, next: the two streams are equal
        emitted = list(t[b, :n]) + [nxt]
        assert emitted == list(am[b, :n + 1])
        if n < K:
            assert t[b, n] != am[b, n]


def test_greedy_config2_by_construction(oracle_mod):
    """Workload 2 plants one substituted token at m_b (m_b = K: none), so
    n = m_b and next = argmax(p_{m_b}) are known from the generator."""
    b = workloads.make_config(2)
    r = oracle_mod.verify_greedy(b.target_probs, b.draft_tokens)
    m = np.array([s["m"] for s in b.info["per_seq"]])
    assert np.array_equal(r["n_accepted"], m)
    am = np.argmax(b.target_probs, axis=2)
    assert np.array_equal(r["next_token"], am[np.arange(b.B), m])
    # all three paths occur: first-token miss, middle miss, full accept
    assert (m == 0).any() and ((m > 0) & (m < b.K)).any() and (m == b.K).any()


def test_greedy_out_of_range_tokens_are_misses(oracle_mod):
    b = workloads.make_batch("c1", 4, 3, 500, seed=3)
    t = np.argmax(b.target_probs[:, :3], axis=2).astype(np.int32)
    t[0, 0] = -1
    t[1, 1] = 500
    t[2, 2] = 2**31 - 1
    r = oracle_mod.verify_greedy(b.target_probs, t)
    assert list(r["n_accepted"]) == [0, 1, 2, 3]


# ------------------------------------------------------ closed forms (P-e) --

@pytest.mark.parametrize("V", [1, 2, 7, 1000, 32000])
def test_k0_greedy_is_argmax(oracle_mod, V):
    rng = np.random.default_rng(V)
    p = rng.random((32, 1, V)).astype(np.float32)
    p[:, :, rng.integers(0, V)] = p.max()      # a tie with a random index
    r = oracle_mod.verify_greedy(p, np.zeros((32, 0), np.int32))
    assert np.array_equal(r["next_token"], np.argmax(p[:, 0], axis=1))
    assert np.all(r["n_accepted"] == 0)


@pytest.mark.parametrize("V", [1, 2, 7, 1000, 32000])
def test_k0_sampled_is_inverse_cdf(oracle_mod, V):
    """K = 0: the draw is plain inverse-CDF sampling of p_0 with u_0, i.e.
    numpy.searchsorted(cumsum(p), u * P, side='right')."""
    rng = np.random.default_rng(100 + V)
    B = 64
    p = (rng.random((B, 1, V)) * (rng.random((B, 1, V)) > 0.3)).astype(np.float32)
    p[:, 0, 0] += np.float32(0.5)
    u = rng.random((B, 1), dtype=np.float32)
    u[0, 0] = 0.0
    r = oracle_mod.verify_sample(p, np.zeros((B, 0, V), np.float32), np.zeros((B, 0), np.int32), u)
    for b in range(B):
        c = np.cumsum(p[b, 0].astype(np.float64))
        x = int(np.searchsorted(c, np.float64(u[b, 0]) * c[-1], side="right"))
        assert int(r["next_token"][b]) == x
    assert np.all(r["n_accepted"] == 0)


def test_q_equals_p_accepts_everything(oracle_mod):
    b = workloads.make_batch("c3", 32, 6, 777, seed=9)
    q = b.target_probs[:, :6].copy()
    rng = np.random.default_rng(1)
    u = rng.random((32, 7), dtype=np.float32)
    u[:, :6] = np.float32(1.0) - np.float32(2.0**-24)   # the largest uniform below 1
    t = np.array([[rng.choice(777, p=q[s, i] / q[s, i].sum()) for i in range(6)] for s in range(32)],
                 np.int32)
    r = oracle_mod.verify_sample(b.target_probs, q, t, u)
    assert np.all(r["n_accepted"] == 6)


def test_one_hot_target_always_emits_its_token(oracle_mod):
    """p_i = s_i * delta(y_i): an accepted draft must be y_i and the final
    token must be y_n, whatever q, t and u are."""
    rng = np.random.default_rng(2)
    B, K, V = 128, 3, 11
    y = rng.integers(0, V, size=(B, K + 1))
    p = np.zeros((B, K + 1, V), np.float32)
    for b in range(B):
        for i in range(K + 1):
            p[b, i, y[b, i]] = np.float32(rng.uniform(0.5, 2.0))
    q = rng.random((B, K, V)).astype(np.float32) + np.float32(0.01)
    t = np.where(rng.random((B, K)) < 0.5, y[:, :K], rng.integers(0, V, size=(B, K))).astype(np.int32)
    u = rng.random((B, K + 1), dtype=np.float32)
    r = oracle_mod.verify_sample(p, q, t, u)
    for b in range(B):
        n = int(r["n_accepted"][b])
        assert list(t[b, :n]) == list(y[b, :n])
        assert int(r["next_token"][b]) == y[b, n]
    assert (r["n_accepted"] > 0).any() and (r["n_accepted"] < K).any()


def test_one_hot_draft(oracle_mod):
    """q_i = s * delta(t_i): accept iff u < p_hat(t); after a rejection the
    draw is from p_hat with t removed (renormalised)."""
    rng = np.random.default_rng(3)
    B, K, V = 256, 2, 9
    p = (rng.random((B, K + 1, V)) + 0.05).astype(np.float32)
    t = rng.integers(0, V, size=(B, K)).astype(np.int32)
    q = np.zeros((B, K, V), np.float32)
    for b in range(B):
        for i in range(K):
            q[b, i, t[b, i]] = np.float32(rng.uniform(0.5, 2.0))
    u = rng.random((B, K + 1), dtype=np.float32)
    r = oracle_mod.verify_sample(p, q, t, u)
    checked = 0
    for b in range(B):
        P = p[b].astype(np.float64).sum(axis=1)
        ph = [p[b, i, t[b, i]] / P[i] for i in range(K)]
        n, near = K, False
        for i in range(K):
            near = abs(u[b, i] - ph[i]) < 1e-9
            if near or not u[b, i] < ph[i]:
                n = i
                break
        if near:
            continue
        assert int(r["n_accepted"][b]) == n
        if n < K:
            w = p[b, n].astype(np.float64).copy()
            w[t[b, n]] = 0.0
            c = np.cumsum(w)
            T = np.float64(u[b, K]) * c[-1]
            if np.min(np.abs(c - T)) < 1e-9 * c[-1]:
                continue
            assert int(r["next_token"][b]) == int(np.searchsorted(c, T, side="right"))
            assert int(r["next_token"][b]) != t[b, n]
        checked += 1
    assert checked > 200


def test_disjoint_supports_reject_first_and_draw_from_p(oracle_mod):
    rng = np.random.default_rng(4)
    B, K, V = 128, 3, 16
    p = np.zeros((B, K + 1, V), np.float32)
    q = np.zeros((B, K, V), np.float32)
    p[:, :, :8] = rng.random((B, K + 1, 8)) + 0.01
    p[:, K, 8:] = rng.random((B, 8)) + 0.01
    q[:, :, 8:] = rng.random((B, K, 8)) + 0.01
    t = rng.integers(8, 16, size=(B, K)).astype(np.int32)
    u = rng.random((B, K + 1), dtype=np.float32)
    r = oracle_mod.verify_sample(p, q, t, u)
    assert np.all(r["n_accepted"] == 0)
    for b in range(B):
        c = np.cumsum(p[b, 0].astype(np.float64))
        T = np.float64(u[b, K]) * c[-1]
        if np.min(np.abs(c - T)) < 1e-9 * c[-1]:
            continue
        assert int(r["next_token"][b]) == int(np.searchsorted(c, T, side="right"))


# ---------------------------------------------------------- masses (P-f) --

@pytest.mark.parametrize("family,V", [("c3", 128256), ("c4", 5000), ("c5", 262144)])
def test_masses_against_fsum(oracle_mod, family, V):
    b = workloads.make_batch(family, 2, 2, V, seed=21)
    r = oracle_mod.verify_sample(b.target_probs, b.draft_probs, b.draft_tokens, b.uniforms)
    st = r["stats"]
    for s in range(2):
        for i in range(3):
            p = b.target_probs[s, i].astype(np.float64)
            P = math.fsum(p)
            assert abs(st["sum_p"][s, i] - P) <= 1e-11 * P
            if i < 2:
                q = b.draft_probs[s, i].astype(np.float64)
                Q = math.fsum(q)
                assert abs(st["sum_q"][s, i] - Q) <= 1e-11 * Q
                smin = math.fsum(np.minimum(p, q))
                spos = math.fsum(np.maximum(p - q, 0.0))
                assert abs(st["sum_min"][s, i] - smin) <= 1e-11 * max(P, Q)
                assert abs(st["sum_pos"][s, i] - spos) <= 1e-11 * max(P, Q)
                # min(p, q) + max(0, p - q) = p, summed
                assert abs(st["sum_min"][s, i] + st["sum_pos"][s, i] - P) <= 1e-11 * P
                t = int(b.draft_tokens[s, i])
                assert st["p_t"][s, i] == b.target_probs[s, i, t]
                assert st["q_t"][s, i] == b.draft_probs[s, i, t]
                # alpha = sum min(p_hat, q_hat)
                a = math.fsum(np.minimum(p / P, q / Q))
                assert abs(r["alpha"][s, i] - a) <= 1e-11


# ------------------------------------------------ preconditions (R10) --

@pytest.mark.parametrize("bad", ["nan", "inf", "neg", "zero_row", "u_one"])
def test_preconditions_raise(oracle_mod, bad):
    b = workloads.make_batch("c1", 1, 2, 64, seed=1)
    p, q, u = b.target_probs.copy(), b.draft_probs.copy(), b.uniforms.copy()
    if bad == "nan":
        p[0, 1, 3] = np.nan
    elif bad == "inf":
        q[0, 0, 5] = np.inf
    elif bad == "neg":
        p[0, 2, 0] = -1e-30
    elif bad == "zero_row":
        q[0, 1, :] = 0
    elif bad == "u_one":
        u[0, 2] = 1.0
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.verify_sample(p, q, b.draft_tokens, u)


# ------------------------------------------- determinism and B-invariance --

def test_threads_and_batch_position_do_not_change_results(oracle_mod):
    b = workloads.make_batch("c3", 24, 5, 3001, seed=8)
    args = (b.target_probs, b.draft_probs, b.draft_tokens, b.uniforms)
    r1 = oracle_mod.verify_sample(*args, threads=1)
    r4 = oracle_mod.verify_sample(*args, threads=4)
    for k in ("n_accepted", "next_token", "stats", "diag", "alpha"):
        assert r1[k].tobytes() == r4[k].tobytes()
    for s in (0, 13, 23):
        one = oracle_mod.verify_sample(*(a[s:s + 1] for a in args))
        assert one["stats"].tobytes() == r1["stats"][s:s + 1].tobytes()
        assert int(one["next_token"][0]) == int(r1["next_token"][s])
