"""Comparison of the HIP library's results with the fp64 oracles.

Bars (the spec-verify kernel card's Method; tolerances from the workload
contract, tightened where the arithmetic allows):
  greedy  - n_accepted, next_token, argmax, max_p and p_t identical (bitwise);
            sum_p within FP64_RTOL relative.
  sampled - argmax, max_p, p_t, q_t identical; P and Q within FP64_RTOL
            relative; sum_min and sum_pos within FP64_RTOL * max(P, Q);
            n_accepted and next_token identical on every sequence whose
            decisions all lie more than BAND_PROB of their mass from a
            boundary (the oracle's margins), and at most
            max(1, MAX_BOUNDARY_FRAC * sequences) sequences exempted.
  logits  - n_accepted and next_token identical outside BAND_LOGITS.

Why these bands.  On probabilities both sides accumulate every mass in fp64
on exactly converted f32 values and differ only in summation order (and the
kernel's published chunk partials give up their 8 lowest mantissa bits,
2^-44 relative): the masses agree to ~V * 2^-53, under 1e-10 relative for
V <= 2^19, and a residual's weights p*Q - q*P inherit that error divided by
the total variation between the rows (>= 0.1 on every workload here).  So a
decision more than 1e-9 of its mass from a boundary is the same on both
sides: BAND_PROB = 1e-9, 10^4 times tighter than the contract's 1e-5.  On
logits the kernel computes each weight in fp32 (exp2 of an fp32 argument,
each about 2^-23 |argument| relative), so a CDF can move by ~1e-6 of its
mass, more for a residual of nearly equal rows: BAND_LOGITS stays at the
contract's 1e-5.
"""
import numpy as np

SUM_RTOL = 1e-5          # the contract
FP64_RTOL = 1e-9         # the check applied to fp64 masses
BAND_CONTRACT = 1e-5
BAND_PROB = 1e-9
BAND_LOGITS = 1e-5
MAX_BOUNDARY_FRAC = 0.01
REPORT_BANDS = (1e-5, 1e-7, 1e-9)


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.maximum(np.abs(b), np.finfo(np.float64).tiny)
    return float(np.max(np.abs(a - b) / den)) if a.size else 0.0


def boundary_mask(diag, band):
    """Sequences with a decision within `band` of its mass from a boundary:
    an acceptance test with |u - ratio| <= band, or a final draw with
    min(T - C(x-1), C(x) - T) <= band * W; and (logits oracle only) a draw
    that took the rounding guard (draw_kind >= 4)."""
    return (diag["accept_margin"] <= band) | (diag["draw_margin"] <= band) | (diag["draw_kind"] >= 4)


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


def compare_outputs(n, nx, orc, band, max_boundary=None, what="sampled"):
    """Identical (n, next) on every sequence outside `band`; at most
    max_boundary sequences inside it (default max(1, 1% of them)).  Returns
    the counts: sequences, boundary (at `band`), boundary_mismatch, and per
    reporting band the sequences inside it and the mismatches among them."""
    d = orc["diag"]
    same = (n == orc["n_accepted"]) & (nx == orc["next_token"])
    bnd = boundary_mask(d, band)
    bad = ~same & ~bnd
    assert not bad.any(), (
        f"{what}: {int(bad.sum())} mismatches outside the {band:g} band; first at "
        f"{int(np.flatnonzero(bad)[0])}: gpu ({int(n[bad][0])}, {int(nx[bad][0])}) oracle "
        f"({int(orc['n_accepted'][bad][0])}, {int(orc['next_token'][bad][0])})")
    out = {"sequences": int(n.size), "band": band, "boundary": int(bnd.sum()),
           "boundary_mismatch": int((~same & bnd).sum())}
    for rb in REPORT_BANDS:
        m = boundary_mask(d, rb)
        out[f"within_{rb:g}"] = int(m.sum())
        out[f"mismatch_within_{rb:g}"] = int((~same & m).sum())
    cap = max(1, int(MAX_BOUNDARY_FRAC * n.size)) if max_boundary is None else max_boundary
    assert out["boundary"] <= cap, f"{what}: {out['boundary']} sequences within the {band:g} band (cap {cap}): {out}"
    return out


def check_sampled(gpu_n, gpu_next, gpu_stats, orc, rows=None, report=None, band=BAND_PROB, max_boundary=None):
    """Returns the counts of compare_outputs."""
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
    out = compare_outputs(n, nx, orc, band, max_boundary)
    if report is not None:
        report.update(out)
    return out


def check_logits(gpu_n, gpu_next, orc, max_boundary=-1):
    """Logits outputs against oracle.logits at BAND_LOGITS.  The 1e-5 band
    holds ~20-35% of final draws at V = 128256, so no cap applies unless
    max_boundary >= 0 is given."""
    cap = gpu_n.size if max_boundary is None or max_boundary < 0 else max_boundary
    return compare_outputs(gpu_n, gpu_next, orc, BAND_LOGITS, cap, what="logits")


def _first_diff(a, b):
    d = np.flatnonzero(np.asarray(a) != np.asarray(b))
    return f"first difference at {d[0]}: {a[d[0]]} vs {b[d[0]]}" if d.size else ""
