"""The C-ABI library builds for gfx950, loads, and exports every function that
include/sv_verify.h declares; host-side argument validation returns its
documented status codes before anything is launched (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sv_verify.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import speculative_decoding_verification_row_amd as sv
    if not os.path.exists(sv.library_path()):
        from speculative_decoding_verification_row_amd import build
        build.build()
    return sv.load_library()


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("sv_verify_greedy_batched", "sv_verify_sample_batched", "sv_workspace_size",
              "sv_workspace_init", "sv_workspace_error", "sv_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    import speculative_decoding_verification_row_amd as sv
    out = subprocess.run(["nm", "-D", "--defined-only", sv.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (sv_[a-z_]+)$", out, flags=re.M))
    for n in _declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)


def test_library_is_built_for_gfx950(lib):
    import speculative_decoding_verification_row_amd as sv
    blob = open(sv.library_path(), "rb").read()
    # the offload bundle names its code-object target
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def test_status_strings(lib):
    import speculative_decoding_verification_row_amd as sv
    assert sv.sv_status_string(0) == "SV_OK"
    for code in (-1, -2, -3, -4, -5):
        assert sv.sv_status_string(code).startswith("SV_ERR_")
    assert "unknown" in sv.sv_status_string(7)


def test_workspace_size(lib):
    import speculative_decoding_verification_row_amd as sv
    small = sv.sv_workspace_size(1, 4, 32000, True)
    big = sv.sv_workspace_size(1024, 8, 128256, True)
    assert 0 < small < big
    assert big < 64 << 20                       # modest: counters and partials only
    assert sv.sv_workspace_size(-1, 4, 100, True) == 0
    assert sv.sv_workspace_size(1, -1, 100, True) == 0
    assert sv.sv_workspace_size(1, 4, 0, True) == 0
    assert sv.sv_workspace_size(1, 4, 524288, True) > 0
    assert sv.sv_workspace_size(1, 4, 524289, True) == 0   # beyond SV_MAX_V
    assert sv.sv_workspace_size(1, 4097, 100, True) == 0   # beyond SV_MAX_K


FAKE = ctypes.c_void_p(0x10000)          # aligned, never dereferenced: calls below return early


def _greedy(lib, tp=FAKE, dt=FAKE, B=1, K=1, V=8, n=FAKE, nx=FAKE, ws=FAKE, wsb=1 << 20, st=None):
    return lib.sv_verify_greedy_batched(tp, dt, B, K, V, n, nx, ws, wsb, st, None)


def _sample(lib, tp=FAKE, dp=FAKE, dt=FAKE, u=FAKE, B=1, K=1, V=8, n=FAKE, nx=FAKE, ws=FAKE,
            wsb=1 << 20, st=None):
    return lib.sv_verify_sample_batched(tp, dp, dt, u, B, K, V, n, nx, ws, wsb, st, None)


def test_argument_errors_greedy(lib):
    assert _greedy(lib, tp=None) == -1
    assert _greedy(lib, dt=None) == -1
    assert _greedy(lib, n=None) == -1
    assert _greedy(lib, nx=None) == -1
    assert _greedy(lib, B=-1) == -1
    assert _greedy(lib, K=-1) == -1
    assert _greedy(lib, V=0) == -1
    assert _greedy(lib, tp=ctypes.c_void_p(0x10002)) == -1          # not 4-byte aligned
    assert _greedy(lib, st=ctypes.c_void_p(0x10004)) == -1          # stats not 8-byte aligned
    assert _greedy(lib, V=524289) == -4
    assert _greedy(lib, K=4097) == -4
    assert _greedy(lib, ws=None) == -2
    assert _greedy(lib, ws=ctypes.c_void_p(0x10008)) == -2          # not 16-byte aligned
    assert _greedy(lib, wsb=16) == -2
    # K = 0 needs no draft tokens; B = 0 is a no-op
    assert _greedy(lib, dt=None, K=0, B=0) == 0
    assert _greedy(lib, B=0) == 0


def test_argument_errors_sampled(lib):
    assert _sample(lib, tp=None) == -1
    assert _sample(lib, dp=None) == -1
    assert _sample(lib, dt=None) == -1
    assert _sample(lib, u=None) == -1
    assert _sample(lib, B=-3) == -1
    assert _sample(lib, V=-5) == -1
    assert _sample(lib, u=ctypes.c_void_p(0x10001)) == -1
    assert _sample(lib, V=600000) == -4
    assert _sample(lib, wsb=0) == -2
    assert _sample(lib, dp=None, dt=None, K=0, B=0) == 0
    assert _sample(lib, B=0) == 0


def test_argument_errors_sampled_early(lib):
    def early(tp=FAKE, dp=FAKE, dt=FAKE, u=FAKE, B=1, K=1, V=8, wsb=1 << 20, ws=FAKE):
        return lib.sv_verify_sample_early_batched(tp, dp, dt, u, B, K, V, FAKE, FAKE, ws, wsb, None)
    assert early(tp=None) == -1
    assert early(dp=None) == -1
    assert early(u=None) == -1
    assert early(B=-3) == -1
    assert early(u=ctypes.c_void_p(0x10001)) == -1
    assert early(V=600000) == -4
    assert early(wsb=0) == -2
    assert early(ws=ctypes.c_void_p(0x10008)) == -2
    assert early(dp=None, dt=None, K=0, B=0) == 0
    assert early(B=0) == 0
    # the logits form: the same checks, and a temperature that is finite and > 0
    def early_l(tau=1.0, tp=FAKE, B=1, K=1, V=8, wsb=1 << 20):
        return lib.sv_verify_sample_logits_early_batched(tp, FAKE, FAKE, FAKE, tau, B, K, V, FAKE, FAKE, FAKE,
                                                         wsb, None)
    assert early_l(tp=None) == -1
    assert early_l(tau=0.0) == -1
    assert early_l(tau=float("nan")) == -1
    assert early_l(wsb=0) == -2
    assert early_l(B=0) == 0


def test_binding_without_library_fails_loudly(monkeypatch, tmp_path):
    import speculative_decoding_verification_row_amd as sv
    monkeypatch.setattr(sv, "_lib", None)
    monkeypatch.setattr(sv, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        sv.load_library()


def _enclosing_function(text, pos):
    """The header line of the top-level function whose body holds `pos`:
    the last line before it that starts a definition at column 0."""
    heads = [m for m in re.finditer(r"^(?:__global__|__device__|static|template|sv_status|extern)[^\n]*$",
                                     text[:pos], flags=re.M)]
    return heads[-1].group(0) if heads else ""


def test_kernel_argument_pointer_is_taken_in_kernel_bodies_only():
    """Inside a called (non-kernel) device function the kernel-argument
    segment pointer is not available: the compiler materialises it as null,
    and a read through it faults.  Every use of the builtin must therefore
    sit in a __global__ function's body, which passes the pointer or the
    values down."""
    src = os.path.join(ROOT, "speculative_decoding_verification_row_amd", "csrc", "sv_verify.hip")
    text = open(src).read()
    uses = [m.start() for m in re.finditer(r"__builtin_amdgcn_kernarg_segment_ptr\s*\(", text)]
    assert uses
    for pos in uses:
        line = text.count("\n", 0, pos) + 1
        if text.rfind("//", text.rfind("\n", 0, pos), pos) >= 0:
            continue                                            # a comment
        head = _enclosing_function(text, pos)
        assert head.startswith("__global__"), f"line {line}: inside `{head}`"


def test_argument_errors_sampled_noalloc(lib):
    """The no-allocation entry point: the sampled call's argument checks, and
    SV_ERR_SCRATCH (-5) for sizes whose workspace exceeds SV_SCRATCH_BYTES,
    all before anything is launched."""
    import speculative_decoding_verification_row_amd as sv

    def na(tp=FAKE, dp=FAKE, dt=FAKE, u=FAKE, B=1, K=1, V=8, n=FAKE, st=None):
        return lib.sv_verify_sample_batched_noalloc(tp, dp, dt, u, B, K, V, n, FAKE, st, None)
    assert na(tp=None) == -1
    assert na(u=None) == -1
    assert na(n=None) == -1
    assert na(B=-1) == -1
    assert na(u=ctypes.c_void_p(0x10001)) == -1
    assert na(V=600000) == -4
    assert na(B=0) == 0
    assert sv.sv_workspace_size(1024, 8, 128256, True) <= sv.SV_SCRATCH_BYTES
    assert sv.sv_workspace_size(1024, 16, 128256, True) > sv.SV_SCRATCH_BYTES
    assert na(B=1024, K=16, V=128256) == -5
    assert "SCRATCH" in sv.sv_status_string(-5)


def test_scratch_size_matches_header():
    import speculative_decoding_verification_row_amd as sv
    text = open(HEADER).read()
    m = re.search(r"#define SV_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == sv.SV_SCRATCH_BYTES


PROBE_HEADER = os.path.join(ROOT, "include", "sv_probe.h")


def test_probe_library_exports_its_header_and_checks_arguments():
    """libsv_probe.so (the streaming-read probe the benchmark reports as
    context) exports what include/sv_probe.h declares; chunk counts and
    argument errors need no GPU."""
    import speculative_decoding_verification_row_amd as sv
    from speculative_decoding_verification_row_amd import build
    path = build.PROBE_LIB
    if not os.path.exists(path):
        build.build()
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(sv_[a-z_]+)\s*\(", text)))
    assert names == ["sv_probe_blocks", "sv_probe_read"]
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (sv_[a-z_]+)$", out, flags=re.M))
    assert set(names) <= exported
    L = ctypes.CDLL(path)
    L.sv_probe_blocks.argtypes = [ctypes.c_size_t, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32]
    L.sv_probe_blocks.restype = ctypes.c_int64
    L.sv_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    assert L.sv_probe_blocks(32768, 32768 + 16, 0, 0) == 3      # one block per started 32 KB chunk
    assert L.sv_probe_blocks(16, 0, 7, 1) == -1                   # unknown mode
    assert L.sv_probe_read(None, 16, None, 0, 0, 0, FAKE, None) == -1
    assert L.sv_probe_read(FAKE, 24, None, 0, 0, 0, FAKE, None) == -1        # size not a multiple of 16
    assert L.sv_probe_read(FAKE, 16, None, 16, 0, 0, FAKE, None) == -1       # second buffer missing
    assert L.sv_probe_read(ctypes.c_void_p(0x10008), 16, None, 0, 0, 0, FAKE, None) == -1   # misaligned
