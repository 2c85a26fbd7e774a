"""Compile the fp64 oracle (oracle/sv_oracle.c) into oracle/libsv_oracle.so.

Test infrastructure: the oracle is built with plain gcc, no -ffast-math and
no floating-point contraction, so every fp64 operation rounds as written.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sv_oracle.c")
LIB = os.path.join(HERE, "libsv_oracle.so")
CMD = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
       "-fno-fast-math", "-pthread", "-Wall", "-Wextra", "-o", LIB, SRC, "-lm"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = CMD[:]
    cmd[cmd.index(LIB)] = tmp
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
