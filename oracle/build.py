"""Compile the fp64 oracle (oracle/sv_oracle.c) into oracle/libsv_oracle.so.

    python oracle/build.py [-v] [--sanitize]

Test infrastructure: the oracle is built with plain gcc, no -ffast-math and
no floating-point contraction, so every fp64 operation rounds as written.
--sanitize builds oracle/libsv_oracle_san.so instead, the same source with
AddressSanitizer and UndefinedBehaviorSanitizer (every report fatal), for a
CPU run of the oracle's pins (tests/test_oracle_sanitized.py); the process
that loads it must preload the sanitizer runtimes (sanitizer_env() gives the
environment).  Neither build involves a GPU.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sv_oracle.c")
LIB = os.path.join(HERE, "libsv_oracle.so")
LIB_SAN = os.path.join(HERE, "libsv_oracle_san.so")
FLAGS = ["-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-pthread", "-Wall", "-Wextra"]
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]
CMD = ["gcc", "-O2"] + FLAGS + ["-o", LIB, SRC, "-lm"]


def command(out: str, sanitize: bool = False) -> list:
    return ["gcc"] + (SAN_FLAGS if sanitize else ["-O2"]) + FLAGS + ["-o", out, SRC, "-lm"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    lib = LIB_SAN if sanitize else LIB
    tmp = lib + ".tmp"
    cmd = command(tmp, sanitize)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def sanitizer_env(base=None) -> dict:
    """Environment for a Python process that loads libsv_oracle_san.so: the
    ASan and UBSan runtimes preloaded, leak checking off (the interpreter
    keeps its allocations until exit), and the oracle's library redirected."""
    def rt(name):
        return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                              check=True).stdout.strip()
    env = dict(os.environ if base is None else base)
    env["LD_PRELOAD"] = f"{rt('libasan.so')}:{rt('libubsan.so')}"
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["SV_ORACLE_LIB"] = LIB_SAN
    return env


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
