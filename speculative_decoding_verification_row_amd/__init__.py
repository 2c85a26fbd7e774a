"""Batched speculative-decoding verification on AMD Instinct MI355X.

Python binding of the C-ABI library libsv_verify.so (include/sv_verify.h).
It marshals torch tensors into device pointers, sizes and a stream, and
calls the library; every step of verification runs in the library's HIP
kernels.  torch provides device memory and streams only.  There is no CPU
path: if the library is not built, importing the binding's entry points
raises.

The operation (the spec-verify kernel card, section "Method"):
  greedy  - accept draft token t_i while it equals the lowest-index argmax of
            target row i; emit that argmax at the first miss, or argmax of
            row K when all K match.
  sampled - accept t_i with probability min(1, p_i(t_i)/q_i(t_i)) on
            row-normalised masses; at the first rejection draw from
            norm(max(0, p_i - q_i)); after full acceptance draw the bonus
            from p_K; uniforms are explicit inputs (u_i for the test of t_i,
            u_K for the final draw).

Names mirror the C ABI: sv_verify_greedy_batched, sv_verify_sample_batched,
sv_workspace_size, sv_workspace_init, sv_workspace_error, sv_status_string.
verify_greedy / verify_sample follow the card's usage, where a 2-D
[K+1, V] target is one sequence.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

__all__ = [
    "SVError", "ROW_STATS_DTYPE", "library_path", "load_library",
    "sv_workspace_size", "sv_workspace_init", "sv_workspace_error", "sv_status_string",
    "sv_verify_greedy_batched", "sv_verify_sample_batched", "sv_verify_sample_early_batched",
    "sv_verify_sample_logits_batched", "sv_verify_sample_logits_early_batched",
    "sv_verify_sample_batched_noalloc", "SV_SCRATCH_BYTES",
    "verify_greedy", "verify_sample", "stats_to_numpy", "workspace_for",
    "SpeculativeDecoder", "DecodeStats", "Governor",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libsv_verify.so")

SV_OK, SV_ERR_INVALID_ARG, SV_ERR_WORKSPACE, SV_ERR_HIP, SV_ERR_UNSUPPORTED, SV_ERR_SCRATCH = 0, -1, -2, -3, -4, -5
SV_SCRATCH_BYTES = 16 << 20   # the library's static device scratch (include/sv_verify.h)

# layout of sv_row_stats (48 bytes)
ROW_STATS_DTYPE = np.dtype([
    ("argmax", np.int32), ("max_p", np.float32),
    ("sum_p", np.float64), ("sum_q", np.float64),
    ("sum_min", np.float64), ("sum_pos", np.float64),
    ("p_t", np.float32), ("q_t", np.float32),
], align=True)
assert ROW_STATS_DTYPE.itemsize == 48


class SVError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {sv_status_string(status)} ({status})")


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libsv_verify.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is not built; run `python -m "
            "speculative_decoding_verification_row_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.sv_workspace_size.argtypes = [I32, I32, I32, I32]
    lib.sv_workspace_size.restype = SZ
    lib.sv_workspace_init.argtypes = [P, SZ, P]
    lib.sv_workspace_init.restype = ctypes.c_int
    lib.sv_verify_greedy_batched.argtypes = [P, P, I32, I32, I32, P, P, P, SZ, P, P]
    lib.sv_verify_greedy_batched.restype = ctypes.c_int
    lib.sv_verify_sample_batched.argtypes = [P, P, P, P, I32, I32, I32, P, P, P, SZ, P, P]
    lib.sv_verify_sample_batched.restype = ctypes.c_int
    lib.sv_verify_sample_early_batched.argtypes = [P, P, P, P, I32, I32, I32, P, P, P, SZ, P]
    lib.sv_verify_sample_early_batched.restype = ctypes.c_int
    lib.sv_verify_sample_logits_batched.argtypes = [P, P, P, P, ctypes.c_float, I32, I32, I32, P, P, P, SZ, P]
    lib.sv_verify_sample_logits_batched.restype = ctypes.c_int
    lib.sv_verify_sample_logits_early_batched.argtypes = [P, P, P, P, ctypes.c_float, I32, I32, I32, P, P, P, SZ, P]
    lib.sv_verify_sample_logits_early_batched.restype = ctypes.c_int
    lib.sv_verify_sample_batched_noalloc.argtypes = [P, P, P, P, I32, I32, I32, P, P, P, P]
    lib.sv_verify_sample_batched_noalloc.restype = ctypes.c_int
    lib.sv_workspace_error.argtypes = [P, ctypes.POINTER(I32), P]
    lib.sv_workspace_error.restype = ctypes.c_int
    lib.sv_status_string.argtypes = [ctypes.c_int]
    lib.sv_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def sv_status_string(status: int) -> str:
    return load_library().sv_status_string(int(status)).decode()


def sv_workspace_size(B: int, K: int, V: int, sampled: bool) -> int:
    return int(load_library().sv_workspace_size(int(B), int(K), int(V), int(bool(sampled))))


def _stream_ptr(stream, device) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(int(stream.cuda_stream))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _call(device_index: int, fn, *args):
    """fn(*args) with `device_index` current (switched only if it is not)."""
    if torch.cuda.current_device() == device_index:
        return fn(*args)
    with torch.cuda.device(device_index):
        return fn(*args)


def _stream_handle(stream, device_index: int) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device_index)
    return int(stream.cuda_stream)


def sv_workspace_init(workspace: torch.Tensor, stream=None) -> None:
    with torch.cuda.device(workspace.device):
        st = load_library().sv_workspace_init(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                              _stream_ptr(stream, workspace.device))
    if st != SV_OK:
        raise SVError(st, "sv_workspace_init")


def sv_workspace_error(workspace: torch.Tensor, stream=None) -> int:
    """Synchronously read the workspace fault word (0 = no fault)."""
    out = ctypes.c_int32(0)
    with torch.cuda.device(workspace.device):
        st = load_library().sv_workspace_error(_ptr(workspace), ctypes.byref(out),
                                               _stream_ptr(stream, workspace.device))
    if st != SV_OK:
        raise SVError(st, "sv_workspace_error")
    return int(out.value)


_WS: dict = {}


_WS_BYTES: dict = {}


def workspace_for(B: int, K: int, V: int, sampled: bool, device, stream=None) -> torch.Tensor:
    """An initialised workspace for (device, stream), grown on demand.  One
    workspace per stream: calls on different streams must not share one."""
    if isinstance(device, int):
        index = device
    else:
        device = torch.device(device)
        index = device.index if device.index is not None else torch.cuda.current_device()
    s = stream if stream is not None else torch.cuda.current_stream(index)
    key = (index, s.cuda_stream)
    shape = (B, K, V, bool(sampled))
    need = _WS_BYTES.get(shape)
    if need is None:
        need = _WS_BYTES[shape] = max(sv_workspace_size(B, K, V, sampled), 256)
    ws = _WS.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=index)
        sv_workspace_init(ws, s)
        _WS[key] = ws
    return ws


def _check(t: torch.Tensor, name: str, dtype, shape: tuple, device_index: int):
    """A contiguous tensor of this dtype and shape on GPU `device_index`: the
    kernels read and write exactly that many elements from its pointer."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype is not dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.shape != shape:
        raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
    if not t.is_cuda or t.get_device() != device_index:
        raise ValueError(f"{name} must be on cuda:{device_index}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _device_of(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a tensor on a HIP device")
    return t.get_device()


def _check_workspace(ws: torch.Tensor, device_index: int):
    """Any contiguous tensor on the call's GPU; its byte size is passed on and
    the library checks it against sv_workspace_size."""
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or ws.get_device() != device_index:
        raise ValueError(f"workspace must be a tensor on cuda:{device_index}")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")


def _outputs(B, device_index, n_accepted, next_token):
    if n_accepted is None:
        n_accepted = torch.empty(B, dtype=torch.int32, device=device_index)
    if next_token is None:
        next_token = torch.empty(B, dtype=torch.int32, device=device_index)
    _check(n_accepted, "n_accepted", torch.int32, (B,), device_index)
    _check(next_token, "next_token", torch.int32, (B,), device_index)
    return n_accepted, next_token


def _stats_buf(stats, B, K, device_index):
    if stats is True:
        stats = torch.empty((B, K + 1, 48), dtype=torch.uint8, device=device_index)
    if stats is None or stats is False:
        return None
    _check(stats, "stats", torch.uint8, (B, K + 1, 48), device_index)
    return stats


def sv_verify_greedy_batched(target_probs: torch.Tensor, draft_tokens: torch.Tensor,
                             n_accepted=None, next_token=None, workspace=None,
                             stats=None, stream=None):
    """Greedy verification of B sequences.

    target_probs [B, K+1, V] float32, draft_tokens [B, K] int32 (CUDA).
    Returns (n_accepted [B] int32, next_token [B] int32[, stats]) on the same
    device; `stats=True` also returns a [B, K+1, 48] uint8 tensor of
    sv_row_stats (see stats_to_numpy)."""
    B, K1, V = target_probs.shape
    K = K1 - 1
    dev = _device_of(target_probs, "target_probs")
    _check(target_probs, "target_probs", torch.float32, (B, K1, V), dev)
    _check(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    n_accepted, next_token = _outputs(B, dev, n_accepted, next_token)
    st = _stats_buf(stats, B, K, dev)
    if workspace is None:
        workspace = workspace_for(B, K, V, False, dev, stream)
    _check_workspace(workspace, dev)
    rc = _call(dev, load_library().sv_verify_greedy_batched,
               target_probs.data_ptr(), draft_tokens.data_ptr(), B, K, V, n_accepted.data_ptr(),
               next_token.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
               None if st is None else st.data_ptr(), _stream_handle(stream, dev))
    if rc != SV_OK:
        raise SVError(rc, "sv_verify_greedy_batched")
    return (n_accepted, next_token, st) if st is not None else (n_accepted, next_token)


def sv_verify_sample_batched(target_probs: torch.Tensor, draft_probs: torch.Tensor,
                             draft_tokens: torch.Tensor, uniforms: torch.Tensor,
                             n_accepted=None, next_token=None, workspace=None,
                             stats=None, stream=None):
    """Sampled verification of B sequences.

    target_probs [B, K+1, V] f32, draft_probs [B, K, V] f32, draft_tokens
    [B, K] int32, uniforms [B, K+1] f32 in [0, 1) (CUDA).  Returns
    (n_accepted, next_token[, stats]) like sv_verify_greedy_batched."""
    B, K1, V = target_probs.shape
    K = K1 - 1
    dev = _device_of(target_probs, "target_probs")
    _check(target_probs, "target_probs", torch.float32, (B, K1, V), dev)
    _check(draft_probs, "draft_probs", torch.float32, (B, K, V), dev)
    _check(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    _check(uniforms, "uniforms", torch.float32, (B, K1), dev)
    n_accepted, next_token = _outputs(B, dev, n_accepted, next_token)
    st = _stats_buf(stats, B, K, dev)
    if workspace is None:
        workspace = workspace_for(B, K, V, True, dev, stream)
    _check_workspace(workspace, dev)
    rc = _call(dev, load_library().sv_verify_sample_batched,
               target_probs.data_ptr(), draft_probs.data_ptr(), draft_tokens.data_ptr(), uniforms.data_ptr(),
               B, K, V, n_accepted.data_ptr(), next_token.data_ptr(),
               workspace.data_ptr(), workspace.numel() * workspace.element_size(),
               None if st is None else st.data_ptr(), _stream_handle(stream, dev))
    if rc != SV_OK:
        raise SVError(rc, "sv_verify_sample_batched")
    return (n_accepted, next_token, st) if st is not None else (n_accepted, next_token)


def sv_verify_sample_early_batched(target_probs: torch.Tensor, draft_probs: torch.Tensor,
                                   draft_tokens: torch.Tensor, uniforms: torch.Tensor,
                                   n_accepted=None, next_token=None, workspace=None, stream=None):
    """Sampled verification with an early exit: the outputs of
    sv_verify_sample_batched bit for bit, reading only the rows they depend
    on (about the pairs 0..n+1 of each sequence, and row K after full
    acceptance).  No row statistics.  Returns (n_accepted, next_token)."""
    B, K1, V = target_probs.shape
    K = K1 - 1
    dev = _device_of(target_probs, "target_probs")
    _check(target_probs, "target_probs", torch.float32, (B, K1, V), dev)
    _check(draft_probs, "draft_probs", torch.float32, (B, K, V), dev)
    _check(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    _check(uniforms, "uniforms", torch.float32, (B, K1), dev)
    n_accepted, next_token = _outputs(B, dev, n_accepted, next_token)
    if workspace is None:
        workspace = workspace_for(B, K, V, True, dev, stream)
    _check_workspace(workspace, dev)
    rc = _call(dev, load_library().sv_verify_sample_early_batched,
               target_probs.data_ptr(), draft_probs.data_ptr(), draft_tokens.data_ptr(), uniforms.data_ptr(),
               B, K, V, n_accepted.data_ptr(), next_token.data_ptr(),
               workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream_handle(stream, dev))
    if rc != SV_OK:
        raise SVError(rc, "sv_verify_sample_early_batched")
    return n_accepted, next_token


def sv_verify_sample_logits_batched(target_logits: torch.Tensor, draft_logits: torch.Tensor,
                                    draft_tokens: torch.Tensor, uniforms: torch.Tensor, temperature: float,
                                    n_accepted=None, next_token=None, workspace=None, stream=None):
    """Sampled verification of B sequences given logits, both warped by
    softmax(l / temperature) inside the library.

    target_logits [B, K+1, V] f32, draft_logits [B, K, V] f32, draft_tokens
    [B, K] int32, uniforms [B, K+1] f32 in [0, 1) (CUDA).  Returns
    (n_accepted, next_token)."""
    B, K1, V = target_logits.shape
    K = K1 - 1
    dev = _device_of(target_logits, "target_logits")
    _check(target_logits, "target_logits", torch.float32, (B, K1, V), dev)
    _check(draft_logits, "draft_logits", torch.float32, (B, K, V), dev)
    _check(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    _check(uniforms, "uniforms", torch.float32, (B, K1), dev)
    n_accepted, next_token = _outputs(B, dev, n_accepted, next_token)
    if workspace is None:
        workspace = workspace_for(B, K, V, True, dev, stream)
    _check_workspace(workspace, dev)
    rc = _call(dev, load_library().sv_verify_sample_logits_batched,
               target_logits.data_ptr(), draft_logits.data_ptr(), draft_tokens.data_ptr(), uniforms.data_ptr(),
               float(temperature), B, K, V, n_accepted.data_ptr(), next_token.data_ptr(),
               workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream_handle(stream, dev))
    if rc != SV_OK:
        raise SVError(rc, "sv_verify_sample_logits_batched")
    return n_accepted, next_token


def sv_verify_sample_logits_early_batched(target_logits: torch.Tensor, draft_logits: torch.Tensor,
                                    draft_tokens: torch.Tensor, uniforms: torch.Tensor, temperature: float,
                                    n_accepted=None, next_token=None, workspace=None, stream=None):
    """Sampled verification on logits with an early exit: the outputs of
    sv_verify_sample_logits_batched bit for bit, reading only the rows they
    depend on.  Same arguments."""
    B, K1, V = target_logits.shape
    K = K1 - 1
    dev = _device_of(target_logits, "target_logits")
    _check(target_logits, "target_logits", torch.float32, (B, K1, V), dev)
    _check(draft_logits, "draft_logits", torch.float32, (B, K, V), dev)
    _check(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    _check(uniforms, "uniforms", torch.float32, (B, K1), dev)
    n_accepted, next_token = _outputs(B, dev, n_accepted, next_token)
    if workspace is None:
        workspace = workspace_for(B, K, V, True, dev, stream)
    _check_workspace(workspace, dev)
    rc = _call(dev, load_library().sv_verify_sample_logits_early_batched,
               target_logits.data_ptr(), draft_logits.data_ptr(), draft_tokens.data_ptr(), uniforms.data_ptr(),
               float(temperature), B, K, V, n_accepted.data_ptr(), next_token.data_ptr(),
               workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream_handle(stream, dev))
    if rc != SV_OK:
        raise SVError(rc, "sv_verify_sample_logits_early_batched")
    return n_accepted, next_token

def sv_verify_sample_batched_noalloc(target_probs: torch.Tensor, draft_probs: torch.Tensor,
                                     draft_tokens: torch.Tensor, uniforms: torch.Tensor,
                                     n_accepted: torch.Tensor, next_token: torch.Tensor,
                                     stats=None, stream=None):
    """sv_verify_sample_batched without a workspace: the library's static
    device scratch serves instead (SV_SCRATCH_BYTES per device).  For callers
    that cannot allocate, the outputs (and a [B, K+1, 48] uint8 stats tensor,
    if wanted) must be preallocated: this binding allocates nothing either.
    Calls that overlap on one device race on the scratch."""
    B, K1, V = target_probs.shape
    K = K1 - 1
    dev = _device_of(target_probs, "target_probs")
    _check(target_probs, "target_probs", torch.float32, (B, K1, V), dev)
    _check(draft_probs, "draft_probs", torch.float32, (B, K, V), dev)
    _check(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    _check(uniforms, "uniforms", torch.float32, (B, K1), dev)
    _check(n_accepted, "n_accepted", torch.int32, (B,), dev)
    _check(next_token, "next_token", torch.int32, (B,), dev)
    if stats is not None:
        _check(stats, "stats", torch.uint8, (B, K1, 48), dev)
    rc = _call(dev, load_library().sv_verify_sample_batched_noalloc,
               target_probs.data_ptr(), draft_probs.data_ptr(), draft_tokens.data_ptr(), uniforms.data_ptr(),
               B, K, V, n_accepted.data_ptr(), next_token.data_ptr(),
               None if stats is None else stats.data_ptr(), _stream_handle(stream, dev))
    if rc != SV_OK:
        raise SVError(rc, "sv_verify_sample_batched_noalloc")
    return n_accepted, next_token


def stats_to_numpy(stats: torch.Tensor) -> np.ndarray:
    """[B, K+1, 48] uint8 device tensor -> [B, K+1] ROW_STATS_DTYPE array."""
    a = stats.detach().cpu().contiguous().numpy()
    return a.view(ROW_STATS_DTYPE).reshape(a.shape[:-1])


def verify_greedy(target_probs, draft_tokens, **kw):
    """The card's `verify_greedy(target_probs [K+1, V], draft_tokens [K])`;
    also accepts batched [B, K+1, V] / [B, K].  Returns (n_accepted,
    next_token) as Python ints for one sequence, tensors for a batch."""
    if target_probs.dim() == 2:
        out = sv_verify_greedy_batched(target_probs.unsqueeze(0), draft_tokens.reshape(1, -1), **kw)
        return int(out[0].item()), int(out[1].item())
    return sv_verify_greedy_batched(target_probs, draft_tokens, **kw)


def verify_sample(target_probs, draft_probs, draft_tokens, uniforms, **kw):
    """Sampled counterpart of verify_greedy; uniforms [K+1] (or [B, K+1])."""
    if target_probs.dim() == 2:
        K = target_probs.shape[0] - 1
        out = sv_verify_sample_batched(target_probs.unsqueeze(0), draft_probs.reshape(1, K, -1),
                                       draft_tokens.reshape(1, -1), uniforms.reshape(1, -1), **kw)
        return int(out[0].item()), int(out[1].item())
    return sv_verify_sample_batched(target_probs, draft_probs, draft_tokens, uniforms, **kw)


# The multi-round driver (the card's SpeculativeDecoder), over the calls above.
from .decoder import DecodeStats, Governor, SpeculativeDecoder  # noqa: E402
