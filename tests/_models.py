"""Synthetic target and draft "models" for the decoder tests.

A model is a deterministic function from a context (a tuple of token ids) to
a next-token distribution over V tokens: logits drawn from N(0, sigma^2) by a
generator seeded with a hash of the context, softmax in fp64, stored as f32.
The draft adds seeded N(0, noise^2) to the target's logits, so it agrees with
the target often but not always (an imperfect draft).  Nothing here knows
the verification method; the tests compare the decoder against plain
decoding of these distributions.
"""
import functools
import hashlib

import numpy as np


def _ctx_key(ctx) -> int:
    h = hashlib.blake2b(np.asarray(ctx, np.int64).tobytes(), digest_size=8).digest()
    return int.from_bytes(h, "little")


class HashLM:
    def __init__(self, V: int, sigma: float = 2.0, salt: int = 1, base=None, noise: float = 0.0):
        self.V, self.sigma, self.salt, self.base, self.noise = V, sigma, salt, base, noise
        self._row = functools.lru_cache(maxsize=1 << 16)(self._row_uncached)

    def logits(self, ctx) -> np.ndarray:
        if self.base is not None:
            g = np.random.default_rng([self.salt, _ctx_key(ctx)])
            return self.base.logits(ctx) + self.noise * g.standard_normal(self.V)
        g = np.random.default_rng([self.salt, _ctx_key(ctx)])
        return self.sigma * g.standard_normal(self.V)

    def _row_uncached(self, ctx: tuple) -> np.ndarray:
        z = self.logits(ctx)
        e = np.exp(z - z.max())
        return (e / e.sum()).astype(np.float32)

    def row(self, ctx) -> np.ndarray:
        """Next-token probabilities after context ctx, f32 [V]."""
        return self._row(tuple(int(t) for t in ctx))


class TiedLM(HashLM):
    """HashLM whose every row copies its maximum to a second, seeded index:
    an exact two-way tie for the argmax (rows are then not normalised, which
    the verifier allows)."""

    def _row_uncached(self, ctx: tuple) -> np.ndarray:
        r = super()._row_uncached(ctx).copy()
        g = np.random.default_rng([self.salt + 7919, _ctx_key(ctx)])
        r[int(g.integers(0, self.V))] = r.max()
        return r


def greedy_decode(model: HashLM, prompt, max_new: int):
    seq = list(prompt)
    for _ in range(max_new):
        seq.append(int(np.argmax(model.row(seq))))
    return seq


def make_callbacks(target: HashLM, draft: HashLM, greedy: bool, seed: int = 0, batched: bool = False):
    """draft_step / target_step in the card's convention (or batched).
    The sampled draft samples its proposals from its own rows with its own
    seeded generator (one draw per proposal, in sequence order)."""
    rng = np.random.default_rng(seed)

    def propose(prefix, k):
        ctx = list(prefix)
        toks, probs = [], []
        for _ in range(k):
            q = draft.row(ctx)
            if greedy:
                t = int(np.argmax(q))
            else:
                c = np.cumsum(q.astype(np.float64))
                t = int(min(np.searchsorted(c, rng.random() * c[-1], side="right"), draft.V - 1))
            toks.append(t)
            probs.append(q)
            ctx.append(t)
        V = draft.V
        return (np.asarray(toks, np.int32).reshape(k),
                np.asarray(probs, np.float32).reshape(k, V))

    def score(prefix, proposed):
        ctx = list(prefix)
        rows = [target.row(ctx)]
        for t in np.asarray(proposed).reshape(-1):
            ctx.append(int(t))
            rows.append(target.row(ctx))
        return np.asarray(rows, np.float32)

    if not batched:
        return propose, score

    def propose_b(prefixes, k):
        out = [propose(p, k) for p in prefixes]
        return np.stack([o[0] for o in out]), np.stack([o[1] for o in out])

    def score_b(prefixes, proposed):
        proposed = np.asarray(proposed).reshape(len(prefixes), -1)
        return np.stack([score(p, proposed[i]) for i, p in enumerate(prefixes)])

    return propose_b, score_b
