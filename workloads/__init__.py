"""Seeded synthetic inputs for the speculative-decoding verification step.

This module builds the operands that a verifier consumes -- target rows
p_i (i = 0..K), draft rows q_i (i < K), draft tokens t_i and explicit
uniforms u_i (i = 0..K) -- with the shapes and value distributions of the
five workload families described below.  It holds none of the verifier's
arithmetic: no acceptance test, no residual and no inverse-CDF draw of the
verification result.  Both the fp64 oracle and the HIP library consume what
it produces, and nothing here imports either of them.

Operand layout (the spec-verify kernel card, "Usage" and "Requirements and
limits"): target_probs [B, K+1, V] f32, draft_probs [B, K, V] f32,
draft_tokens [B, K] int32, uniforms [B, K+1] f32 in [0, 1).

Every sequence b is drawn from its own PCG64 stream seeded by
SeedSequence([seed, family, round, b]), so any single sequence of a batch can
be regenerated alone (the oracle's bounded samples rely on this).

Families (shapes are the defaults of the five workloads; tests shrink them):

  c1  B=1,   K=4,  V=32000.  logits ~ N(0, 2^2), p = softmax(logits);
      q = softmax(logits + SIGMA_C1 * N(0, 1)) with SIGMA_C1 fixed by
      bisection so that the mean per-token acceptance sum(min(p, q)) is 0.68
      (workloads/calibrate_c1.py reproduces the value); t ~ q; u ~ U[0, 1).
  c2  B=64,  K=4,  V=32000, greedy only.  logits ~ N(0, 3^2); t_i = argmax
      p_i except at one position m_b ~ U{0..K} (m_b = K: none) where a token
      drawn uniformly from V minus {argmax} is substituted.
  c3  B=256, K=5,  V=128256.  logits ~ N(0, 2.5^2); sigma_b ~ U[0.3, 2.0] per
      sequence; q = softmax(logits + sigma_b * N(0, 1)); t ~ q.
  c4  B=1024, K=8, V=128256, unnormalized.  As c3, then every p row and every
      q row is multiplied (in f32) by its own scale ~ U[0.5, 2]; a seeded
      quarter of the sequences (exactly B // 4) use q_i := scaled p_i bitwise
      and t_i ~ p_i.
  c5  B=32,  K=16, V=262144.  Zipf(s=1.1) rows over a per-row seeded token
      permutation; in 10% of p rows the maximum is copied to 1-3 more indices
      (2-4-way exact ties) before an fp64 renormalisation; q_i is the same law
      over the permutation of p_i with 20% of its ranks reshuffled among
      themselves; t ~ q.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

# Mean per-token acceptance sum(min(p, q)) of 0.68 for family c1 at V=32000
# (logits N(0, 2^2)); reproduced by workloads/calibrate_c1.py.
SIGMA_C1 = 0.8243408203125

FAMILIES = ("c1", "c2", "c3", "c4", "c5")
_FAMILY_ID = {f: i + 1 for i, f in enumerate(FAMILIES)}

# Default shapes of the five workloads, and which modes each one runs.
CONFIGS = {
    1: dict(family="c1", B=1, K=4, V=32000, modes=("greedy", "sampled"), rounds=600),
    2: dict(family="c2", B=64, K=4, V=32000, modes=("greedy",), rounds=1),
    3: dict(family="c3", B=256, K=5, V=128256, modes=("sampled",), rounds=1),
    4: dict(family="c4", B=1024, K=8, V=128256, modes=("sampled",), rounds=1),
    5: dict(family="c5", B=32, K=16, V=262144, modes=("greedy", "sampled"), rounds=1),
}


@dataclass
class Batch:
    """One batch of verifier operands (host numpy arrays)."""
    family: str
    B: int
    K: int
    V: int
    seed: int
    rnd: int
    target_probs: np.ndarray            # [B, K+1, V] f32
    draft_probs: np.ndarray | None      # [B, K, V] f32 (None for c2)
    draft_tokens: np.ndarray            # [B, K] int32
    uniforms: np.ndarray                # [B, K+1] f32
    info: dict = field(default_factory=dict)

    def sha256(self) -> str:
        h = hashlib.sha256()
        for a in (self.target_probs, self.draft_probs, self.draft_tokens, self.uniforms):
            if a is not None:
                h.update(np.ascontiguousarray(a).tobytes())
        return h.hexdigest()


def _rng(seed: int, family: str, rnd: int, b: int) -> np.random.Generator:
    ss = np.random.SeedSequence([seed, _FAMILY_ID[family], rnd, b])
    return np.random.Generator(np.random.PCG64(ss))


def _softmax_f32(logits: np.ndarray) -> np.ndarray:
    """fp64 softmax of one row, stored as f32 (input construction only)."""
    z = logits.astype(np.float64)
    z -= z.max()
    e = np.exp(z)
    e /= e.sum()
    return e.astype(np.float32)


def _draw_index(rng: np.random.Generator, row_f32: np.ndarray) -> int:
    """Draw one token from the normalised f32 row (input construction only)."""
    c = np.cumsum(row_f32.astype(np.float64))
    r = rng.random() * c[-1]
    return int(min(np.searchsorted(c, r, side="right"), row_f32.size - 1))


_ZIPF_CACHE: dict[int, np.ndarray] = {}


def _zipf_weights(V: int) -> np.ndarray:
    w = _ZIPF_CACHE.get(V)
    if w is None:
        w = np.arange(1, V + 1, dtype=np.float64) ** -1.1
        _ZIPF_CACHE[V] = w
    return w


def _c4_qeqp_set(seed: int, rnd: int, B: int) -> np.ndarray:
    """Exactly B // 4 sequence indices of a c4 batch that use q = p."""
    ss = np.random.SeedSequence([seed, _FAMILY_ID["c4"], rnd, 0x7FFFFFFF, B])
    rng = np.random.Generator(np.random.PCG64(ss))
    mask = np.zeros(B, dtype=bool)
    mask[rng.choice(B, size=B // 4, replace=False)] = True
    return mask


def gen_sequence(family: str, b: int, B: int, K: int, V: int, seed: int = 0, rnd: int = 0,
                 out_p: np.ndarray | None = None, out_q: np.ndarray | None = None, logits: bool = False):
    """Generate sequence b of a batch.

    Returns (p [K+1, V] f32, q [K, V] f32 or None, t [K] int32, u [K+1] f32, info).
    If out_p / out_q are given, the rows are written there (and returned).
    logits=True (families c1, c3): the rows are the f32 logits themselves, not
    their softmax, and the draft tokens are drawn from the softmax of the
    stored draft logits (temperature 1); the random draws are those of the
    probability rows.
    """
    if logits and family not in ("c1", "c3"):
        raise ValueError(f"family {family} has no logits form")
    if family not in _FAMILY_ID:
        raise ValueError(f"unknown family {family!r}")
    rng = _rng(seed, family, rnd, b)
    p = out_p if out_p is not None else np.empty((K + 1, V), dtype=np.float32)
    q = None
    if family != "c2":
        q = out_q if out_q is not None else np.empty((K, V), dtype=np.float32)
    t = np.empty(K, dtype=np.int32)
    info: dict = {}

    if family in ("c1", "c3", "c4"):
        scale = {"c1": 2.0, "c3": 2.5, "c4": 2.5}[family]
        if family == "c1":
            sigma = SIGMA_C1
        else:
            sigma = float(rng.uniform(0.3, 2.0))
        info["sigma"] = sigma
        qeqp = False
        if family == "c4":
            qeqp = bool(_c4_qeqp_set(seed, rnd, B)[b])
            info["q_equals_p"] = qeqp
        for i in range(K + 1):
            z = scale * rng.standard_normal(V)
            if logits:
                p[i] = z.astype(np.float32)
                if i < K:
                    q[i] = (z + sigma * rng.standard_normal(V)).astype(np.float32)
                continue
            p[i] = _softmax_f32(z)
            if i < K:
                q[i] = _softmax_f32(z + sigma * rng.standard_normal(V))
        if family == "c4":
            sp = rng.uniform(0.5, 2.0, size=K + 1).astype(np.float32)
            sq = rng.uniform(0.5, 2.0, size=K).astype(np.float32)
            for i in range(K + 1):
                p[i] *= sp[i]
            for i in range(K):
                if qeqp:
                    q[i] = p[i]
                else:
                    q[i] *= sq[i]
        for i in range(K):
            t[i] = _draw_index(rng, _softmax_f32(q[i]) if logits else q[i])
    elif family == "c2":
        for i in range(K + 1):
            p[i] = _softmax_f32(3.0 * rng.standard_normal(V))
        m = int(rng.integers(0, K + 1))
        info["m"] = m
        for i in range(K):
            a = int(np.argmax(p[i]))
            if i == m:
                r = int(rng.integers(0, V - 1))
                t[i] = r if r < a else r + 1
            else:
                t[i] = a
    elif family == "c5":
        w = _zipf_weights(V)
        ties = []
        perms = []
        for i in range(K + 1):
            perm = rng.permutation(V)
            perms.append(perm)
            row = np.empty(V, dtype=np.float64)
            row[perm] = w
            k = 1
            if rng.random() < 0.1:
                k = int(rng.integers(2, 5))
                top = int(perm[0])
                others = rng.choice(V - 1, size=k - 1, replace=False)
                others = others + (others >= top)
                row[others] = row[top]
            ties.append(k)
            p[i] = (row / row.sum()).astype(np.float32)
        info["tie_ways"] = ties
        for i in range(K):
            perm = perms[i].copy()
            m = int(round(0.2 * V))
            ranks = rng.choice(V, size=m, replace=False)
            perm[ranks] = perm[rng.permutation(ranks)]
            row = np.empty(V, dtype=np.float64)
            row[perm] = w
            q[i] = (row / row.sum()).astype(np.float32)
            t[i] = _draw_index(rng, q[i])
    u = rng.random(K + 1, dtype=np.float32)
    return p, q, t, u, info


def make_batch(family: str, B: int, K: int, V: int, seed: int = 0, rnd: int = 0,
               seqs=None, logits: bool = False) -> Batch:
    """Generate a whole batch (or only the sequences listed in `seqs`, which
    then become rows 0..len(seqs)-1 of the returned arrays)."""
    idx = list(range(B)) if seqs is None else [int(s) for s in seqs]
    n = len(idx)
    tp = np.empty((n, K + 1, V), dtype=np.float32)
    dp = None if family == "c2" else np.empty((n, K, V), dtype=np.float32)
    dt = np.empty((n, K), dtype=np.int32)
    u = np.empty((n, K + 1), dtype=np.float32)
    infos = []
    for j, b in enumerate(idx):
        _, _, t, uu, info = gen_sequence(family, b, B, K, V, seed, rnd,
                                         out_p=tp[j], out_q=None if dp is None else dp[j], logits=logits)
        dt[j] = t
        u[j] = uu
        infos.append(info)
    return Batch(family, B, K, V, seed, rnd, tp, dp, dt, u,
                 {"seqs": idx, "per_seq": infos})


def make_config(cfg: int, seed: int = 0, rnd: int = 0, seqs=None, **override) -> Batch:
    """Batch of workload `cfg` (1..5) with its default shape; keyword
    overrides (B, K, V) shrink it for tests."""
    c = dict(CONFIGS[cfg])
    c.update(override)
    return make_batch(c["family"], c["B"], c["K"], c["V"], seed=seed, rnd=rnd, seqs=seqs)


def formula_bytes(B: int, K: int, V: int, sampled: bool) -> int:
    """Bytes every verification round must stream: (K+1)*V*4 per sequence,
    plus K*V*4 when the draft rows are read (sampled mode)."""
    per = (K + 1) * V * 4 + (K * V * 4 if sampled else 0)
    return B * per


def _gen_one(args):
    family, b, B, K, V, seed, rnd, logits = args
    p, q, t, u, info = gen_sequence(family, b, B, K, V, seed, rnd, logits=logits)
    return b, p, q, t, u, info


def iter_sequences(family: str, B: int, K: int, V: int, seed: int = 0, rnd: int = 0,
                   seqs=None, workers: int = 1, logits: bool = False):
    """Yield (b, p, q, t, u, info) for each requested sequence, in order,
    generating them in `workers` forked processes when workers > 1."""
    idx = list(range(B)) if seqs is None else [int(s) for s in seqs]
    jobs = [(family, b, B, K, V, seed, rnd, logits) for b in idx]
    if workers <= 1 or len(jobs) <= 1:
        for j in jobs:
            yield _gen_one(j)
        return
    import multiprocessing as mp
    ctx = mp.get_context("fork")
    with ctx.Pool(processes=workers) as pool:
        for r in pool.imap(_gen_one, jobs, chunksize=1):
            yield r


def default_workers() -> int:
    """Worker processes for generation: the CPUs this process may use, capped
    at 16."""
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))
