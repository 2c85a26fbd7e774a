"""Place a generated batch directly in device memory (torch tensors), one
sequence at a time, so that the host never holds the whole batch."""
from __future__ import annotations

import hashlib

import numpy as np

from . import CONFIGS, iter_sequences, default_workers


def device_batch(family: str, B: int, K: int, V: int, seed: int = 0, rnd: int = 0,
                 device="cuda", workers: int | None = None, sampled: bool = True,
                 keep_host=None, logits: bool = False, progress=None):
    """Return dict(tp, dp, dt, u) of device tensors plus 'info' (per-sequence
    generator info) and 'sha256' of the host bytes.  keep_host: optional set
    of sequence indices whose host arrays are also returned in 'host'.
    progress: optional callable(done, B), called every 128 sequences."""
    import torch
    workers = default_workers() if workers is None else workers
    tp = torch.empty((B, K + 1, V), dtype=torch.float32, device=device)
    dp = torch.empty((B, K, V), dtype=torch.float32, device=device) if sampled else None
    dt = np.empty((B, K), np.int32)
    u = np.empty((B, K + 1), np.float32)
    infos = [None] * B
    host = {}
    h = hashlib.sha256()
    pin_p = torch.empty((K + 1, V), dtype=torch.float32, pin_memory=True)
    pin_q = torch.empty((max(K, 1), V), dtype=torch.float32, pin_memory=True)
    for b, p, q, t, uu, info in iter_sequences(family, B, K, V, seed, rnd, workers=workers, logits=logits):
        pin_p.numpy()[...] = p
        tp[b].copy_(pin_p, non_blocking=False)
        h.update(p.tobytes())
        if sampled:
            if q is None:
                raise ValueError(f"family {family} has no draft rows")
            if K:
                pin_q[:K].numpy()[...] = q
                dp[b].copy_(pin_q[:K], non_blocking=False)
            h.update(q.tobytes())
        dt[b] = t
        u[b] = uu
        infos[b] = info
        if keep_host is not None and b in keep_host:
            host[b] = (p, q, t, uu)
        if progress is not None and (b + 1) % 128 == 0:
            progress(b + 1, B)
    h.update(dt.tobytes())
    h.update(u.tobytes())
    return {
        "tp": tp, "dp": dp,
        "dt": torch.from_numpy(dt).to(device), "u": torch.from_numpy(u).to(device),
        "dt_host": dt, "u_host": u, "info": infos, "host": host, "sha256": h.hexdigest(),
    }


def device_config(cfg: int, seed: int = 0, rnd: int = 0, device="cuda", sampled=None, **kw):
    c = dict(CONFIGS[cfg])
    if sampled is None:
        sampled = "sampled" in c["modes"]
    return device_batch(c["family"], c["B"], c["K"], c["V"], seed, rnd, device, sampled=sampled, **kw)
