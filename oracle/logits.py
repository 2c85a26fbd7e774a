"""fp64 oracle of sampled verification on logits with a temperature.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It never imports the
HIP library.

The spec-verify kernel card's speculative-sampling bullet (section
"Method") is distribution-preserving when the target and draft distributions
are warped identically, and its requirements make that warping the caller's
job.  Given logits instead, this oracle warps both with one temperature tau
(reading: the warped distribution of a row of logits l is softmax(l / tau)):
each row's weights are w(x) = exp((l(x) - max l) / tau) in fp64, and its
mass is their ascending sequential sum.  Verification then takes the steps
of the probability oracle (sv_oracle.c) on these fp64 weights:
  accept t_i iff u_i * q_i(t_i) * P_i < p_i(t_i) * Q_i (scale-free);
  n = the first rejected row, else K;
  n < K: residual weights max(0, p_n * Q_n - q_n * P_n) (p_n when their
  total is 0); n == K: the weights of row K;
  next = the smallest x whose running sum exceeds u_K * (total), else (by
  rounding only) the last x with positive weight.
A draft token outside [0, V) has zero weight on both sides and is rejected.

The last rule (the rounding guard) is reachable only when the searched
total W is below fp64's normal range: for a normal W, u_K * W rounds below W
(u_K <= 1 - 2^-24), and the running sum reaches W at the last position.  A
residual can be that small only when every position where the target
outweighs the draft has a weight below about 2^-1000, e.g. a target logit
745 * tau under its row's maximum against a draft weight of 0.
"""
from __future__ import annotations

import numpy as np

from . import SEQ_DIAG_DTYPE, OracleError


def warp_row(logits_row, tau: float) -> np.ndarray:
    """fp64 weights exp((l - max l) / tau) of one row of f32 logits."""
    z = np.asarray(logits_row, np.float32).astype(np.float64)
    return np.exp((z - z.max()) / float(tau))


def _seq_sum(w: np.ndarray) -> float:
    """Ascending sequential fp64 sum (the order every oracle sum uses)."""
    return float(np.cumsum(w)[-1]) if w.size else 0.0


def verify_sample_logits(target_logits, draft_logits, draft_tokens, uniforms, temperature) -> dict:
    """target_logits [B, K+1, V] f32, draft_logits [B, K, V] f32,
    draft_tokens [B, K] int32, uniforms [B, K+1] f32, temperature > 0.
    Returns dict(n_accepted [B], next_token [B], diag [B] SEQ_DIAG_DTYPE,
    P [B, K+1], Q [B, K] the rows' masses, M [B, K+1], MQ [B, K] their
    maxima)."""
    tl = np.ascontiguousarray(target_logits, np.float32)
    B, K1, V = tl.shape
    K = K1 - 1
    dl = np.ascontiguousarray(draft_logits, np.float32).reshape(B, K, V)
    dt = np.ascontiguousarray(draft_tokens, np.int32).reshape(B, K)
    u = np.ascontiguousarray(uniforms, np.float32).reshape(B, K1)
    tau = float(np.float32(temperature))
    if not (np.isfinite(tau) and tau > 0.0):
        raise OracleError("temperature must be finite and > 0")
    if V < 1 or not np.all(np.isfinite(tl)) or not np.all(np.isfinite(dl)):
        raise OracleError("logits must be finite")
    if np.any((u < 0) | (u >= 1)):
        raise OracleError("uniforms must lie in [0, 1)")
    n_out = np.empty(B, np.int32)
    x_out = np.empty(B, np.int32)
    dg = np.zeros(B, SEQ_DIAG_DTYPE)
    Pm = np.zeros((B, K1))
    Qm = np.zeros((B, K))
    Mm = tl.max(axis=2).astype(np.float64) if V else np.zeros((B, K1))
    MQ = dl.max(axis=2).astype(np.float64) if K else np.zeros((B, 0))
    for b in range(B):
        wp = [warp_row(tl[b, i], tau) for i in range(K1)]
        wq = [warp_row(dl[b, i], tau) for i in range(K)]
        P = [_seq_sum(w) for w in wp]
        Q = [_seq_sum(w) for w in wq]
        Pm[b], Qm[b] = P, Q
        n, acc_margin = K, np.inf
        for i in range(K):
            t = int(dt[b, i])
            tin = 0 <= t < V
            pt = wp[i][t] if tin else 0.0
            qt = wq[i][t] if tin else 0.0
            lhs = float(u[b, i]) * qt * P[i]
            rhs = pt * Q[i]
            if qt * P[i] > 0.0:
                acc_margin = min(acc_margin, abs(lhs - rhs) / (qt * P[i]))
            if not (lhs < rhs):
                n = i
                break
        if n < K:
            kind = 1
            w = np.maximum(wp[n] * Q[n] - wq[n] * P[n], 0.0)
            if _seq_sum(w) == 0.0:
                kind, w = 3, wp[n]
        else:
            kind, w = 2, wp[K]
        c = np.cumsum(w)
        W = float(c[-1])
        T = float(u[b, K]) * W
        x = int(np.searchsorted(c, T, side="right"))
        if x >= V:                       # rounding guard
            x = int(np.flatnonzero(w > 0.0)[-1])
            kind += 4
            dmargin = 0.0
        else:
            lo = T - (float(c[x - 1]) if x > 0 else 0.0)
            dmargin = min(lo, float(c[x]) - T) / W
        n_out[b], x_out[b] = n, x
        dg[b] = (n, x, n, kind, acc_margin, dmargin, W, T)
    return {"n_accepted": n_out, "next_token": x_out, "diag": dg, "P": Pm, "Q": Qm, "M": Mm, "MQ": MQ}
