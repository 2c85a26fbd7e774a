"""Comparison of the HIP library's results with the fp64 oracle.

Bars (the spec-verify kernel card's Method; tolerances from the workload
contract):
  greedy  - n_accepted, next_token, argmax, max_p and p_t identical (bitwise);
            sum_p within SUM_RTOL relative.
  sampled - argmax, max_p, p_t, q_t identical; P and Q within SUM_RTOL
            relative; sum_min and sum_pos within SUM_RTOL * max(P, Q);
            n_accepted and next_token identical on every sequence whose
            decisions all lie more than BAND (1e-5) of their mass from a
            boundary (the oracle's margins); boundary sequences are counted
            and reported.
Both sides accumulate masses in fp64 on exactly converted f32 values; they
differ only in summation order, so sums agree to ~V * 2^-53 relative.
SUM_RTOL = 1e-5 is the contract; FP64_RTOL = 1e-9 is the check actually
applied, far tighter (the order difference is below 1e-10 for V <= 2^19).
"""
import numpy as np

SUM_RTOL = 1e-5
FP64_RTOL = 1e-9
BAND = 1e-5


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.maximum(np.abs(b), np.finfo(np.float64).tiny)
    return float(np.max(np.abs(a - b) / den)) if a.size else 0.0


def check_greedy(gpu_n, gpu_next, gpu_stats, orc, rows=None):
    """gpu_* are numpy arrays; orc is the oracle's verify_greedy result.
    rows: optional index array selecting the oracle's sequences in the GPU batch."""
    sel = slice(None) if rows is None else rows
    n, nx = gpu_n[sel], gpu_next[sel]
    assert np.array_equal(n, orc["n_accepted"]), _first_diff(n, orc["n_accepted"])
    assert np.array_equal(nx, orc["next_token"]), _first_diff(nx, orc["next_token"])
    if gpu_stats is not None:
        g, o = gpu_stats[sel], orc["stats"]
        assert np.array_equal(g["argmax"], o["argmax"])
        assert g["max_p"].tobytes() == o["max_p"].tobytes()
        assert g["p_t"].tobytes() == o["p_t"].tobytes()
        assert _rel(g["sum_p"], o["sum_p"]) <= FP64_RTOL
        for f in ("sum_q", "sum_min", "sum_pos", "q_t"):
            assert not np.any(g[f]), f


def boundary_mask(orc):
    d = orc["diag"]
    return (d["accept_margin"] <= BAND) | (d["draw_margin"] <= BAND) | (d["draw_kind"] >= 4)


def check_sampled(gpu_n, gpu_next, gpu_stats, orc, rows=None, report=None):
    """Returns dict(boundary=..., boundary_mismatch=..., n=...)."""
    sel = slice(None) if rows is None else rows
    n, nx = gpu_n[sel], gpu_next[sel]
    if gpu_stats is not None:
        g, o = gpu_stats[sel], orc["stats"]
        assert np.array_equal(g["argmax"], o["argmax"])
        assert g["max_p"].tobytes() == o["max_p"].tobytes()
        assert g["p_t"].tobytes() == o["p_t"].tobytes()
        assert g["q_t"].tobytes() == o["q_t"].tobytes()
        P, Q = o["sum_p"], o["sum_q"]
        assert _rel(g["sum_p"], P) <= FP64_RTOL
        K1 = P.shape[1]
        if K1 > 1:
            assert _rel(g["sum_q"][:, :-1], Q[:, :-1]) <= FP64_RTOL
            scale = np.maximum(P, Q)[:, :-1]
            for f in ("sum_min", "sum_pos"):
                err = np.abs(g[f][:, :-1] - o[f][:, :-1]) / scale
                assert float(err.max()) <= FP64_RTOL, f
        for f in ("sum_q", "sum_min", "sum_pos", "q_t", "p_t"):
            assert not np.any(g[f][:, -1]), f
    bnd = boundary_mask(orc)
    same = (n == orc["n_accepted"]) & (nx == orc["next_token"])
    bad = ~same & ~bnd
    assert not bad.any(), (
        f"{int(bad.sum())} non-boundary mismatches; first at {int(np.flatnonzero(bad)[0])}: "
        f"gpu ({int(n[bad][0])}, {int(nx[bad][0])}) oracle "
        f"({int(orc['n_accepted'][bad][0])}, {int(orc['next_token'][bad][0])})")
    out = {"sequences": int(n.size), "boundary": int(bnd.sum()),
           "boundary_mismatch": int((~same & bnd).sum())}
    if report is not None:
        report.update(out)
    return out


def _first_diff(a, b):
    d = np.flatnonzero(np.asarray(a) != np.asarray(b))
    return f"first difference at {d[0]}: {a[d[0]]} vs {b[d[0]]}" if d.size else ""
