"""Pins of the oracle's decision margins, its zero-residual fallback (R8) and
the inverse CDF's termination.

The margins decide which sequences a GPU parity test may exempt as boundary
sequences, so they are pinned here against an independent recomputation:
row masses by math.fsum (correctly rounded), each acceptance ratio by plain
division, rho_i = (p_i(t_i)/P_i) / (q_i(t_i)/Q_i), and the final draw by
numpy.cumsum plus numpy.searchsorted.  The accept margin of a sequence is the
smallest |u_i - rho_i| over the tests it performed (a test whose q(t) is 0
adds none), the draw margin is min(T - C(x-1), C(x) - T) / W at the drawn x.
Hand-derived margins of small dyadic cases are in tests/golden.

R8 (spec-verify kernel card, section "Method", speculative-sampling bullet:
the residual is norm(max(0, p - q))): a rejection whose residual has no mass
draws from the rejected row's target p_n.  That happens exactly when the
rows agree after normalisation, e.g. q_n equal to p_n bit for bit (or 2 p_n)
with a rejected draft token that lies outside [0, V) or has p(t) = q(t) = 0.
The draw is then plain inverse-CDF sampling of p_n with u_K:
numpy.searchsorted(cumsum(p_n), u_K * P_n, side='right').

Termination: the oracle never needs a rounding guard; sv_oracle.c proves that
some x has C(x) > T for valid inputs and returns an error otherwise.  These
tests drive it with the largest uniform below 1 on rows of extreme scales.
"""
import math

import numpy as np
import pytest

import workloads

F64 = np.float64
U_MAX = np.float32(1.0) - np.float32(2.0 ** -24)   # the largest f32 below 1


def _independent(p, q, t, u):
    """One sequence: (n, next, draw_kind, accept_margin, draw_margin, W, T)."""
    K1, V = p.shape
    K = K1 - 1
    P = [math.fsum(p[i].astype(F64)) for i in range(K1)]
    Q = [math.fsum(q[i].astype(F64)) for i in range(K)]
    n, am = K, math.inf
    for i in range(K):
        ti = int(t[i])
        tin = 0 <= ti < V
        pt = float(p[i, ti]) if tin else 0.0
        qt = float(q[i, ti]) if tin else 0.0
        if qt > 0.0:
            rho = (pt / P[i]) / (qt / Q[i])
            am = min(am, abs(float(u[i]) - rho))
            accept = float(u[i]) < rho
        else:
            accept = pt > 0.0          # u * 0 < p(t) * Q
        if not accept:
            n = i
            break
    if n < K:
        w = np.maximum(p[n].astype(F64) * Q[n] - q[n].astype(F64) * P[n], 0.0)
        kind = 1
        if not np.any(w > 0.0):
            w, kind = p[n].astype(F64), 3
    else:
        w, kind = p[K].astype(F64), 2
    c = np.cumsum(w)
    W = float(c[-1])
    T = float(u[K]) * W
    x = int(np.searchsorted(c, T, side="right"))
    lo = T - (float(c[x - 1]) if x > 0 else 0.0)
    hi = float(c[x]) - T
    return n, x, kind, am, min(lo, hi) / W, W, T, w


def _random_rows(rng, B, K, V, scale_exp=0):
    """Uniform rows with 20% zeros and planted ties, tokens half at the
    argmax and half uniform (a few out of range), optional power-of-two
    scale."""
    p = rng.random((B, K + 1, V)).astype(np.float32)
    q = rng.random((B, K, V)).astype(np.float32)
    p[rng.random(p.shape) < 0.2] = 0
    q[rng.random(q.shape) < 0.2] = 0
    p[..., 0] += np.float32(1e-3)
    q[..., -1] += np.float32(1e-3)
    if scale_exp:
        p = (p * np.float32(2.0 ** scale_exp)).astype(np.float32)
        q = (q * np.float32(2.0 ** (scale_exp // 2))).astype(np.float32)
    t = np.where(rng.random((B, K)) < 0.5, np.argmax(p[:, :K], axis=2),
                 rng.integers(-2, V + 2, size=(B, K))).astype(np.int32)
    u = rng.random((B, K + 1), dtype=np.float32)
    return p, q, t, u


def _cases():
    out = []
    for fam, B, K, V in [("c1", 24, 4, 4000), ("c3", 32, 5, 3001), ("c4", 32, 8, 2500), ("c5", 8, 16, 4096)]:
        b = workloads.make_batch(fam, B, K, V, seed=31)
        out.append((f"{fam}", b.target_probs, b.draft_probs, b.draft_tokens, b.uniforms))
    rng = np.random.default_rng(77)
    for V, sc in [(7, 0), (300, 0), (1000, -140), (1000, 100)]:
        out.append((f"random V={V} scale 2^{sc}",) + _random_rows(rng, 48, 3, V, sc))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c[0])
def test_margins_against_independent_recomputation(oracle_mod, case):
    _, p, q, t, u = case
    r = oracle_mod.verify_sample(p, q, t, u)
    d = r["diag"]
    checked = 0
    for s in range(p.shape[0]):
        n, x, kind, am, dm, W, T, _ = _independent(p[s], q[s], t[s], u[s])
        # the margins agree wherever they are defined, boundary or not
        if math.isinf(am):
            assert math.isinf(d["accept_margin"][s])
        else:
            assert abs(d["accept_margin"][s] - am) <= 1e-12, (s, d["accept_margin"][s], am)
        if am <= 1e-9:
            continue        # the independent ratio may decide the other way
        assert int(r["n_accepted"][s]) == n and int(d["draw_kind"][s]) == kind
        assert abs(d["W"][s] - W) <= 1e-12 * W and abs(d["T"][s] - T) <= 1e-12 * W
        assert abs(d["draw_margin"][s] - dm) <= 1e-12, (s, d["draw_margin"][s], dm)
        if dm <= 1e-9:
            continue
        assert int(r["next_token"][s]) == x
        checked += 1
    assert checked >= 0.95 * p.shape[0]


def test_margins_locate_planted_boundaries(oracle_mod):
    """A uniform placed at distance e from the acceptance ratio (or from a
    CDF breakpoint) yields a margin of e: the margins measure what the parity
    tests use them for."""
    rng = np.random.default_rng(5)
    B, K, V = 64, 1, 64
    p = (rng.random((B, 2, V)) + 0.01).astype(np.float32)
    q = (rng.random((B, 1, V)) + 0.01).astype(np.float32)
    t = rng.integers(0, V, size=(B, 1)).astype(np.int32)
    u = rng.random((B, 2), dtype=np.float32)
    eps = np.float32(2.0 ** -12)
    for s in range(B):
        P, Q = math.fsum(p[s, 0].astype(F64)), math.fsum(q[s, 0].astype(F64))
        rho = (float(p[s, 0, t[s, 0]]) / P) / (float(q[s, 0, t[s, 0]]) / Q)
        if rho < 1.0:
            u[s, 0] = np.float32(rho) + eps          # rejected, margin ~ eps
    r = oracle_mod.verify_sample(p, q, t, u)
    d = r["diag"]
    for s in range(B):
        _, _, _, am, dm, _, _, _ = _independent(p[s], q[s], t[s], u[s])
        assert abs(d["accept_margin"][s] - am) <= 1e-12
        if u[s, 0] > 0.0 and abs(am - float(eps)) < 2.0 ** -24:
            assert int(r["n_accepted"][s]) == 0
    # the draw: T placed just past a breakpoint of the bonus row
    p2 = np.full((1, 1, 8), 0.125, np.float32)
    for k, want in [(3, 3), (5, 5)]:
        uk = np.float32(k / 8 + 2.0 ** -20)
        r = oracle_mod.verify_sample(p2, np.zeros((1, 0, 8), np.float32), np.zeros((1, 0), np.int32),
                                     np.array([[uk]], np.float32))
        assert int(r["next_token"][0]) == want
        assert abs(r["diag"]["draw_margin"][0] - 2.0 ** -20) <= 1e-15


def _r8_batch(rng, variant, B=48, K=5, V=3001, fam="c3"):
    b = workloads.make_batch(fam, B, K, V, seed=int(rng.integers(1 << 30)))
    p, q = b.target_probs.copy(), b.draft_probs.copy()
    t, u = b.draft_tokens.copy(), b.uniforms.copy()
    nsel = rng.integers(0, K, size=B)
    for s in range(B):
        n = int(nsel[s])
        for i in range(n):                       # certain acceptance
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
    return p, q, t, u, nsel


@pytest.mark.parametrize("variant", ["out_of_range_low", "out_of_range_high", "zero_mass_token", "scaled_copy"])
def test_r8_zero_residual_draws_from_target_row(oracle_mod, variant):
    rng = np.random.default_rng(hash(variant) % (1 << 31))
    p, q, t, u, nsel = _r8_batch(rng, variant)
    K = q.shape[1]
    r = oracle_mod.verify_sample(p, q, t, u)
    for s in range(p.shape[0]):
        n = int(nsel[s])
        c = np.cumsum(p[s, n].astype(F64))
        x = int(np.searchsorted(c, F64(u[s, K]) * c[-1], side="right"))
        assert int(r["n_accepted"][s]) == n
        assert int(r["diag"]["draw_kind"][s]) == 3
        assert int(r["next_token"][s]) == x
        assert r["diag"]["W"][s] == c[-1]


@pytest.mark.parametrize("scale", [0, -140, 110])
def test_inverse_cdf_always_finds_a_token(oracle_mod, scale):
    """u_K = 1 - 2^-24 on rows of ordinary, subnormal and huge scale, with
    residual, bonus and R8 draws: the oracle returns a token (it would raise
    otherwise), the token carries weight, and it is the last token with
    weight whenever that token holds more than 2^-23 of the mass."""
    rng = np.random.default_rng(1000 + scale)
    p, q, t, u = _random_rows(rng, 64, 3, 500, scale)
    p[:8, :, 1:] = 0                               # single-token rows
    u[:, -1] = U_MAX
    r = oracle_mod.verify_sample(p, q, t, u)
    kinds = set()
    for s in range(p.shape[0]):
        n, _, kind, am, _, W, _, w = _independent(p[s], q[s], t[s], u[s])
        if am <= 1e-9:
            continue
        kinds.add(kind)
        x = int(r["next_token"][s])
        assert w[x] > 0.0
        last = int(np.flatnonzero(w > 0.0)[-1])
        if w[last] > 2.0 ** -23 * W:
            assert x == last
    assert {1, 2} <= kinds
