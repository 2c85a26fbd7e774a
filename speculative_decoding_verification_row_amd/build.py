"""Build libsv_verify.so (the C-ABI library) and libsv_probe.so (the
streaming-read probe the benchmark reports as context) for gfx950 with hipcc,
in-tree.

    python -m speculative_decoding_verification_row_amd.build [-v]

The command is kept here (not in a Makefile) so the build step the tests,
benchmark and smoke check rely on is one importable function.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "sv_verify.hip")
LIB = os.path.join(PKG, "libsv_verify.so")
# the streaming-read probe the benchmark reports as context (not the method)
PROBE_SRC = os.path.join(PKG, "csrc", "sv_probe.hip")
PROBE_LIB = os.path.join(PKG, "libsv_probe.so")
INCLUDE = os.path.join(ROOT, "include")
ARCH = os.environ.get("SV_OFFLOAD_ARCH", "gfx950")


def command(out: str, src: str = SRC) -> list:
    return ["hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-function",
            # packed fp32 instructions are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-o", out, src]


def build(verbose: bool = False) -> str:
    """Build the library and the probe; returns the library's path."""
    _build_one(SRC, LIB, verbose)
    _build_one(PROBE_SRC, PROBE_LIB, verbose)
    return LIB


def _build_one(src: str, lib: str, verbose: bool) -> str:
    tmp = lib + ".tmp"
    cmd = command(tmp, src)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name; that
    # warning is expected and harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if l.strip() and noise not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
