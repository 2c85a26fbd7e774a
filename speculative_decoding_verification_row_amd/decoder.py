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

The verification itself always runs in the library's HIP kernels; `verify`
replaces it only for tests that exercise this host protocol without a GPU.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, List, Optional, Sequence

import numpy as np
import torch

from . import sv_verify_greedy_batched, sv_verify_sample_batched, workspace_for


@dataclass
class DecodeStats:
    """Per-round record of a generate call: rounds run, and for every
    (round, sequence) the number of drafts accepted."""
    rounds: int = 0
    accepted: List[int] = field(default_factory=list)

    def mean_accepted(self) -> float:
        return float(np.mean(self.accepted)) if self.accepted else 0.0

    def histogram(self, k: int) -> np.ndarray:
        return np.bincount(np.asarray(self.accepted, np.int64), minlength=k + 1)


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
    verify    -- test hook: callable(tp, dp, tokens, uniforms) -> (n, next)
                 on numpy arrays of one round, replacing the library call.
    """

    def __init__(self, draft_step: Callable, target_step: Callable, k: int = 4, greedy: bool = True,
                 seed: int = 0, device=None, batched: bool = False, verify: Optional[Callable] = None):
        if k < 0:
            raise ValueError("k must be >= 0")
        self.draft_step = draft_step
        self.target_step = target_step
        self.k = int(k)
        self.greedy = bool(greedy)
        self.batched = bool(batched)
        self.verify = verify
        self.device = device
        self.rng = np.random.Generator(np.random.PCG64(seed))
        self.stats = DecodeStats()

    # one round for the sequences whose prefixes are given
    def _round(self, prefixes: List[List[int]]):
        b, k = len(prefixes), self.k
        if self.batched:
            toks, dprobs = self.draft_step(prefixes, k)
            tprobs = self.target_step(prefixes, toks)
        else:
            toks, dprobs = self.draft_step(prefixes[0], k)
            tprobs = self.target_step(prefixes[0], toks)
        u = self.rng.random((b, k + 1), dtype=np.float32)
        if self.verify is not None:   # test hook: host arrays of the round
            tp = np.asarray(torch.as_tensor(tprobs).cpu(), np.float32).reshape(b, k + 1, -1)
            tk = np.asarray(torch.as_tensor(toks).cpu(), np.int32).reshape(b, k)
            dp = None if self.greedy else np.asarray(torch.as_tensor(dprobs).cpu(), np.float32).reshape(b, k, -1)
            n, nx = self.verify(tp, dp, tk, u)
            return np.asarray(tk), np.asarray(n), np.asarray(nx)
        dev = torch.device(self.device) if self.device is not None else torch.device("cuda", torch.cuda.current_device())
        tp = torch.as_tensor(tprobs, device=dev)
        V = tp.shape[-1]
        tp = _as_f32(tp, dev, (b, k + 1, V))
        tk = _as_int32(toks, dev, (b, k))
        ws = workspace_for(b, k, V, not self.greedy, dev)
        if self.greedy:
            n, nx = sv_verify_greedy_batched(tp, tk, workspace=ws)
        else:
            dp = _as_f32(dprobs, dev, (b, k, V))
            ut = torch.from_numpy(u).to(dev, non_blocking=False)
            n, nx = sv_verify_sample_batched(tp, dp, tk, ut, workspace=ws)
        # one transfer back (it waits for the round's kernels)
        host = torch.cat([tk.reshape(-1), n, nx]).cpu().numpy()
        return host[:b * k].reshape(b, k), host[b * k:b * k + b], host[b * k + b:]

    def generate_many(self, prompts: Sequence[Sequence[int]], max_new: int = 128,
                      stop_token: Optional[int] = None) -> List[List[int]]:
        """Every prompt followed by its generated tokens (at most max_new;
        generation also ends after stop_token)."""
        if not self.batched and len(prompts) != 1:
            raise ValueError("unbatched callbacks take one prompt; construct with batched=True")
        seqs = [list(map(int, p)) for p in prompts]
        new = [0] * len(seqs)
        done = [max_new <= 0] * len(seqs)
        while not all(done):
            active = [i for i, d in enumerate(done) if not d]
            toks, n, nx = self._round([seqs[i] for i in active])
            self.stats.rounds += 1
            for j, i in enumerate(active):
                nj = int(n[j])
                self.stats.accepted.append(nj)
                emitted = [int(t) for t in toks[j, :nj]] + [int(nx[j])]
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
