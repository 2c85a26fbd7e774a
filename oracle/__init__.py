"""Python access to the fp64 CPU oracle (oracle/sv_oracle.c).

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It never imports the
HIP library, and the HIP library never imports it.

The oracle computes the verification step of the spec-verify kernel card
(section "Method"): greedy verification (accept while the draft token equals
the target row's argmax) and speculative sampling (accept with probability
min(1, p/q) on row-normalised masses, residual norm(max(0, p - q)) on the
first rejection, bonus from p_K after full acceptance), in fp64 with
ascending-index sums.  The conventions it fixes where the card is silent are
listed at the top of sv_oracle.c.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SV_ORACLE_LIB selects another build of the same source (the sanitizer
# build of oracle/build.py --sanitize).
_LIB_PATH = os.environ.get("SV_ORACLE_LIB") or os.path.join(_HERE, "libsv_oracle.so")

ROW_STATS_DTYPE = np.dtype([
    ("argmax", np.int32), ("max_p", np.float32),
    ("sum_p", np.float64), ("sum_q", np.float64),
    ("sum_min", np.float64), ("sum_pos", np.float64),
    ("p_t", np.float32), ("q_t", np.float32),
], align=True)

SEQ_DIAG_DTYPE = np.dtype([
    ("n_accepted", np.int32), ("next_token", np.int32),
    ("draw_row", np.int32), ("draw_kind", np.int32),
    ("accept_margin", np.float64), ("draw_margin", np.float64),
    ("W", np.float64), ("T", np.float64),
], align=True)

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    lib.svo_verify_greedy.argtypes = [P, P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int64,
                                      P, P, P, ctypes.c_int32]
    lib.svo_verify_greedy.restype = ctypes.c_int
    lib.svo_verify_sample.argtypes = [P, P, P, P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int64,
                                      P, P, P, P, P, ctypes.c_int32]
    lib.svo_verify_sample.restype = ctypes.c_int
    lib.svo_sizeof_row_stats.restype = ctypes.c_int32
    lib.svo_sizeof_seq_diag.restype = ctypes.c_int32
    assert lib.svo_sizeof_row_stats() == ROW_STATS_DTYPE.itemsize
    assert lib.svo_sizeof_seq_diag() == SEQ_DIAG_DTYPE.itemsize
    _lib = lib
    return lib


class OracleError(ValueError):
    pass


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _prep(tp, dt, dp=None, u=None):
    tp = np.ascontiguousarray(tp, dtype=np.float32)
    if tp.ndim == 2:            # [K+1, V] -> B = 1
        tp = tp[None]
        dt = np.asarray(dt)[None]
        if dp is not None:
            dp = np.asarray(dp)[None]
        if u is not None:
            u = np.asarray(u)[None]
    B, K1, V = tp.shape
    K = K1 - 1
    dt = np.ascontiguousarray(dt, dtype=np.int32).reshape(B, K)
    if dp is not None:
        dp = np.ascontiguousarray(dp, dtype=np.float32).reshape(B, K, V)
    if u is not None:
        u = np.ascontiguousarray(u, dtype=np.float32).reshape(B, K + 1)
    return tp, dt, dp, u, B, K, V


def verify_greedy(target_probs, draft_tokens, threads: int = 1) -> dict:
    """Greedy verification.  Returns dict(n_accepted [B], next_token [B],
    stats [B, K+1] structured ROW_STATS_DTYPE)."""
    tp, dt, _, _, B, K, V = _prep(target_probs, draft_tokens)
    n = np.empty(B, np.int32)
    nxt = np.empty(B, np.int32)
    st = np.zeros((B, K + 1), ROW_STATS_DTYPE)
    rc = _load().svo_verify_greedy(_ptr(tp), _ptr(dt), B, K, V, _ptr(n), _ptr(nxt), _ptr(st),
                                   int(threads))
    if rc != 0:
        raise OracleError(f"oracle greedy: precondition violated (rc={rc})")
    return {"n_accepted": n, "next_token": nxt, "stats": st}


def verify_sample(target_probs, draft_probs, draft_tokens, uniforms, threads: int = 1,
                  diagnostics: bool = True) -> dict:
    """Sampled verification.  Returns dict(n_accepted, next_token, and when
    diagnostics=True also stats [B, K+1], diag [B] (SEQ_DIAG_DTYPE) and
    alpha [B, K], the normalised per-row acceptance sum_x min(p/P, q/Q))."""
    tp, dt, dp, u, B, K, V = _prep(target_probs, draft_tokens, draft_probs, uniforms)
    n = np.empty(B, np.int32)
    nxt = np.empty(B, np.int32)
    st = np.zeros((B, K + 1), ROW_STATS_DTYPE) if diagnostics else None
    dg = np.zeros(B, SEQ_DIAG_DTYPE) if diagnostics else None
    al = np.zeros((B, K), np.float64) if diagnostics else None
    rc = _load().svo_verify_sample(_ptr(tp), _ptr(dp), _ptr(dt), _ptr(u), B, K, V,
                                   _ptr(n), _ptr(nxt), _ptr(st), _ptr(dg), _ptr(al),
                                   int(threads))
    if rc == -4:
        raise OracleError("oracle sampled: the inverse CDF found no token, which the proof in "
                          "sv_oracle.c rules out for valid inputs")
    if rc != 0:
        raise OracleError(f"oracle sampled: precondition violated (rc={rc})")
    out = {"n_accepted": n, "next_token": nxt}
    if diagnostics:
        out.update(stats=st, diag=dg, alpha=al)
    return out


def expected_accepted_length(alpha_row: np.ndarray) -> tuple[float, float]:
    """Mean and variance of n_accepted for one sequence whose K per-row
    acceptance probabilities are alpha_row (tests are independent):
    P(n >= i) = prod_{j < i} alpha_j, so E[n] = sum_{i=1..K} prod_{j<i} alpha_j."""
    K = len(alpha_row)
    surv = np.cumprod(np.concatenate([[1.0], np.asarray(alpha_row, np.float64)]))  # P(n >= i), i=0..K
    probs = np.empty(K + 1)
    for i in range(K):
        probs[i] = surv[i] * (1.0 - alpha_row[i])
    probs[K] = surv[K]
    ks = np.arange(K + 1)
    mean = float((ks * probs).sum())
    var = float((ks * ks * probs).sum() - mean * mean)
    return mean, var
