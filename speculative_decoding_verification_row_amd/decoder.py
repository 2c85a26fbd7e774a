"""Multi-round speculative decoding driver over the verification library.

The spec-verify kernel card (section "Usage", the SpeculativeDecoder lines,
and section "API") drives the whole draft/verify loop from two user
callbacks:

  draft_step(prefix, k)            -> (tokens [k], probs [k, V])
  target_step(prefix, proposed)    -> target_probs [k+1, V]

Row j of target_probs is the target's distribution after prefix followed by
proposed[:j].  Each round verifies the k proposals with one call of the
library (greedy or sampled, section "Method"); the accepted prefix of the
proposals and the one correction or bonus token the call emits are appended,
and that token is the pending token the next round's draft continues from.
Greedy rounds need no draft probabilities (the draft may return None for
them) and make the emitted stream identical to plain greedy decoding of the
target.  Sampled rounds draw their k+1 uniforms from the decoder's seeded
generator, so a seed fixes the whole stream given the callbacks.

With batched=True the callbacks receive a list of prefixes (one per active
sequence) and return tokens [b, k], probs [b, k, V] and target_probs
[b, k+1, V]; a round then verifies every active sequence in one launch, and a
sequence leaves the batch once it has max_new tokens (or emitted the stop
token).

Telemetry and the governor follow the SPEL README (section 1.3, the Dynamic
Speculation Governor, and its definition of the acceptance fraction as
accepted draft tokens over proposed ones; corrections and bonus tokens are
delivered output, not accepted drafts).  A Governor, per sequence, keeps the
accepted/proposed ratio over a window of its last rounds; when that ratio
falls below alpha_threshold, or a round accepts none of its proposals, the
sequence stops drafting for the rest of the generate call and continues one
target token per round (a K = 0 verification: plain greedy or sampled
target decoding).  It does not resume drafting within the call.

forced_alpha (benchmark only, as the llms-explorer post's forced-acceptance
ceilings): the drafts and the verification run for real, then the accepted
prefix is replaced by a run of Bernoulli(forced_alpha) successes drawn from
the decoder's generator, followed by the argmax of the target row after it.
That argmax is the library's own (lowest index on ties): a forcing round asks
its verification call for the row statistics, whose argmax field holds every
target row's.  The output is then not a decoding of the target.

The verification itself always runs in the library's HIP kernels; `verify`
replaces it only for tests that exercise this host protocol without a GPU
(in a forcing round the hook also returns every target row's argmax).
"""
from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field
from typing import Callable, List, Optional, Sequence

import numpy as np
import torch

from . import sv_verify_greedy_batched, sv_verify_sample_batched, sv_verify_sample_early_batched, workspace_for


@dataclass
class DecodeStats:
    """Telemetry of a decoder: rounds run; for every drafting (round,
    sequence) the drafts accepted; per draft position, how often it was
    tested and accepted; governor trips and the target-only rounds after
    them."""
    rounds: int = 0
    accepted: List[int] = field(default_factory=list)
    proposed: int = 0
    position_tested: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    position_accepted: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    trips: int = 0
    ar_rounds: int = 0

    def record(self, k: int, n: int) -> None:
        if self.position_tested.size < k:
            grow = k - self.position_tested.size
            self.position_tested = np.concatenate([self.position_tested, np.zeros(grow, np.int64)])
            self.position_accepted = np.concatenate([self.position_accepted, np.zeros(grow, np.int64)])
        self.accepted.append(n)
        self.proposed += k
        self.position_tested[:min(n + 1, k)] += 1
        self.position_accepted[:n] += 1

    def mean_accepted(self) -> float:
        return float(np.mean(self.accepted)) if self.accepted else 0.0

    def acceptance_fraction(self) -> float:
        """Accepted draft tokens over proposed ones."""
        return float(np.sum(self.accepted)) / self.proposed if self.proposed else 0.0

    def position_rate(self) -> np.ndarray:
        """Per draft position: accepted over tested."""
        t = self.position_tested
        return np.where(t > 0, self.position_accepted / np.maximum(t, 1), 0.0)

    def histogram(self, k: int) -> np.ndarray:
        return np.bincount(np.asarray(self.accepted, np.int64), minlength=k + 1)


@dataclass
class Governor:
    """Stop drafting when the accepted/proposed ratio over the last `window`
    drafting rounds falls below alpha_threshold, or (trip_on_zero) when a
    round accepts none of its proposals."""
    alpha_threshold: float = 0.0
    window: int = 8
    trip_on_zero: bool = True


class _GovState:
    def __init__(self, g: Governor):
        self.g = g
        self.hist = deque(maxlen=max(1, int(g.window)))
        self.tripped = False

    def update(self, n: int, k: int) -> bool:
        """Record a drafting round; True if the governor trips now."""
        self.hist.append((n, k))
        acc = sum(a for a, _ in self.hist)
        prop = sum(p for _, p in self.hist)
        if (self.g.trip_on_zero and k > 0 and n == 0) or (prop > 0 and acc / prop < self.g.alpha_threshold):
            self.tripped = True
        return self.tripped


def _as_int32(x, device, shape) -> torch.Tensor:
    t = torch.as_tensor(x, device=device).to(torch.int32).reshape(shape)
    return t.contiguous()


def _as_f32(x, device, shape) -> torch.Tensor:
    t = torch.as_tensor(x, device=device)
    if t.dtype != torch.float32:
        raise TypeError(f"probabilities must be float32, got {t.dtype}")
    return t.reshape(shape).contiguous()


class SpeculativeDecoder:
    """SpeculativeDecoder(draft_step, target_step, k=4, greedy=True).

    seed      -- seeds the generator of the sampled rounds' uniforms.
    device    -- device of the verification (default: the current one).
    batched   -- callbacks take and return batches (see the module notes).
    governor  -- a Governor (per sequence, reset by every generate call).
    forced_alpha -- benchmark only: force the accepted prefix (see above).
    verify    -- test hook: callable(tp, dp, tokens, uniforms) -> (n, next)
                 on numpy arrays of one round, replacing the library call;
                 with forced_alpha it returns (n, next, argmax [b, k+1]).
    """

    def __init__(self, draft_step: Callable, target_step: Callable, k: int = 4, greedy: bool = True,
                 seed: int = 0, device=None, batched: bool = False, verify: Optional[Callable] = None,
                 governor: Optional[Governor] = None, forced_alpha: Optional[float] = None):
        if k < 0:
            raise ValueError("k must be >= 0")
        if forced_alpha is not None and not (0.0 <= forced_alpha <= 1.0):
            raise ValueError("forced_alpha must lie in [0, 1]")
        self.governor = governor
        self.forced_alpha = forced_alpha
        self.draft_step = draft_step
        self.target_step = target_step
        self.k = int(k)
        self.greedy = bool(greedy)
        self.batched = bool(batched)
        self.verify = verify
        self.device = device
        self.rng = np.random.Generator(np.random.PCG64(seed))
        self.stats = DecodeStats()
        self._bufcache: dict = {}

    # one round of k proposals (k == 0: target only) for the given prefixes;
    # returns (tokens [b, k], n [b], next [b], argmax of the target rows
    # [b, k+1] when forcing, else None)
    def _round(self, prefixes: List[List[int]], k: int):
        b = len(prefixes)
        if k == 0:
            toks, dprobs = np.zeros((b, 0), np.int32), None
        elif self.batched:
            toks, dprobs = self.draft_step(prefixes, k)
        else:
            toks, dprobs = self.draft_step(prefixes[0], k)
        if self.batched:
            tprobs = self.target_step(prefixes, toks)
        else:
            tprobs = self.target_step(prefixes[0], toks if k else [])
        u = self.rng.random((b, k + 1), dtype=np.float32)
        forcing = self.forced_alpha is not None and k > 0
        if self.verify is not None:   # test hook: host arrays of the round
            tp = np.asarray(torch.as_tensor(tprobs).cpu(), np.float32).reshape(b, k + 1, -1)
            tk = np.asarray(torch.as_tensor(toks).cpu(), np.int32).reshape(b, k)
            V = tp.shape[-1]
            dp = None if self.greedy else (np.zeros((b, 0, V), np.float32) if k == 0 else
                                           np.asarray(torch.as_tensor(dprobs).cpu(), np.float32).reshape(b, k, V))
            res = self.verify(tp, dp, tk, u)
            if forcing and len(res) != 3:
                raise ValueError("with forced_alpha the verify hook returns (n, next, row argmax)")
            am = np.asarray(res[2]).reshape(b, k + 1) if forcing else None
            return np.asarray(tk), np.asarray(res[0]), np.asarray(res[1]), am
        dev = self._device()
        tp = torch.as_tensor(tprobs, device=dev)
        V = tp.shape[-1]
        tp = _as_f32(tp, dev, (b, k + 1, V))
        host_toks = None if isinstance(toks, torch.Tensor) else np.asarray(toks, np.int32).reshape(b, k)
        tk = _as_int32(toks, dev, (b, k))
        bufs = self._buffers(dev, b, k, V, forcing)
        stream, ws = bufs["stream"], bufs["ws"]
        o = b * k
        dev_out, host_out = bufs["dev"], bufs["host"]
        st = bufs.get("stats")   # forcing: every target row's argmax, from the row statistics
        if self.greedy:
            sv_verify_greedy_batched(tp, tk, n_accepted=bufs["n"], next_token=bufs["x"], workspace=ws,
                                     stats=st, stream=stream)
        else:
            dp = (torch.zeros((b, 0, V), dtype=torch.float32, device=dev) if k == 0 else
                  _as_f32(dprobs, dev, (b, k, V)))
            bufs["u_host"][...] = u
            bufs["u_dev"].copy_(bufs["u_pin"], non_blocking=True)
            if forcing:
                sv_verify_sample_batched(tp, dp, tk, bufs["u_dev"], n_accepted=bufs["n"], next_token=bufs["x"],
                                         workspace=ws, stats=st, stream=stream)
            else:
                # the early exit: the full pass's outputs, bit for bit,
                # reading only the rows they depend on
                sv_verify_sample_early_batched(tp, dp, tk, bufs["u_dev"], n_accepted=bufs["n"],
                                               next_token=bufs["x"], workspace=ws, stream=stream)
        if host_toks is None:
            dev_out[:o].copy_(tk.reshape(-1))
        if forcing:
            # the argmax field (the first int32 of each 48-byte sv_row_stats)
            dev_out[o + 2 * b:].copy_(st.view(torch.int32).reshape(b, k + 1, 12)[:, :, 0].reshape(-1))
        # one transfer back into pinned memory, then wait for the round's work
        host_out.copy_(dev_out, non_blocking=True)
        stream.synchronize()
        h = bufs["host_np"]
        am = h[o + 2 * b:].reshape(b, k + 1).copy() if forcing else None
        tks = host_toks if host_toks is not None else h[:o].reshape(b, k).copy()
        return tks, h[o:o + b].copy(), h[o + b:o + 2 * b].copy(), am

    def _device(self) -> torch.device:
        if self.device is not None:
            return torch.device(self.device)
        return torch.device("cuda", torch.cuda.current_device())

    def _buffers(self, dev, b: int, k: int, V: int, forcing: bool) -> dict:
        """Per (device, stream, b, k, V): a device int32 buffer for the
        round's tokens, n, next (and argmaxes) with views of n and next, its
        pinned host mirror, pinned and device uniforms, the stream, the
        verification workspace and, when forcing, the row statistics."""
        stream = torch.cuda.current_stream(dev)
        key = (dev.index, stream.cuda_stream, b, k, V, forcing)
        bufs = self._bufcache.get(key)
        if bufs is None:
            size = b * k + 2 * b + (b * (k + 1) if forcing else 0)
            o = b * k
            bufs = {"dev": torch.empty(size, dtype=torch.int32, device=dev),
                    "host": torch.empty(size, dtype=torch.int32, pin_memory=True),
                    "u_pin": torch.empty((b, k + 1), dtype=torch.float32, pin_memory=True),
                    "u_dev": torch.empty((b, k + 1), dtype=torch.float32, device=dev),
                    "stream": stream,
                    "ws": workspace_for(b, k, V, not self.greedy, dev, stream)}
            if forcing:
                bufs["stats"] = torch.empty((b, k + 1, 48), dtype=torch.uint8, device=dev)
            bufs["n"], bufs["x"] = bufs["dev"][o:o + b], bufs["dev"][o + b:o + 2 * b]
            bufs["host_np"] = bufs["host"].numpy()
            bufs["u_host"] = bufs["u_pin"].numpy()
            self._bufcache[key] = bufs
        return bufs

    def generate_many(self, prompts: Sequence[Sequence[int]], max_new: int = 128,
                      stop_token: Optional[int] = None) -> List[List[int]]:
        """Every prompt followed by its generated tokens (at most max_new;
        generation also ends after stop_token)."""
        if not self.batched and len(prompts) != 1:
            raise ValueError("unbatched callbacks take one prompt; construct with batched=True")
        seqs = [list(map(int, p)) for p in prompts]
        new = [0] * len(seqs)
        done = [max_new <= 0] * len(seqs)
        gov = [_GovState(self.governor) if self.governor is not None else None for _ in seqs]
        while not all(done):
            active = [i for i, d in enumerate(done) if not d]
            drafting = [i for i in active if not (gov[i] and gov[i].tripped)] if self.k > 0 else []
            plain = [i for i in active if i not in set(drafting)]
            self.stats.rounds += 1
            for group, k in ((drafting, self.k), (plain, 0)):
                if not group:
                    continue
                toks, n, nx, am = self._round([seqs[i] for i in group], k)
                if k == 0 and self.k > 0:
                    self.stats.ar_rounds += len(group)
                for j, i in enumerate(group):
                    nj = int(n[j])
                    emitted = [int(t) for t in toks[j, :nj]] + [int(nx[j])]
                    if am is not None:   # forced prefix (benchmark only)
                        nf = 0
                        while nf < k and self.rng.random() < self.forced_alpha:
                            nf += 1
                        nj = nf
                        emitted = [int(t) for t in toks[j, :nf]] + [int(am[j, nf])]
                    if k > 0:
                        self.stats.record(k, nj)
                        if gov[i] is not None and not gov[i].tripped and gov[i].update(nj, k):
                            self.stats.trips += 1
                    for t in emitted:
                        seqs[i].append(t)
                        new[i] += 1
                        if new[i] >= max_new or (stop_token is not None and t == stop_token):
                            done[i] = True
                            break
        return seqs

    def generate(self, prompt_ids, max_new: int = 128, stop_token: Optional[int] = None):
        """The card's dec.generate(prompt_ids, max_new): the prompt followed by
        the generated tokens, as a list of ints (a list of such lists when
        batched and given several prompts)."""
        if self.batched:
            if len(prompt_ids) and isinstance(prompt_ids[0], (list, tuple, np.ndarray, torch.Tensor)):
                return self.generate_many(prompt_ids, max_new, stop_token)
            return self.generate_many([prompt_ids], max_new, stop_token)[0]
        if isinstance(prompt_ids, torch.Tensor):
            prompt_ids = prompt_ids.reshape(-1).tolist()
        return self.generate_many([prompt_ids], max_new, stop_token)[0]
