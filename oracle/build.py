"""Compile the C oracle into ``oracle/libgqa_oracle.so`` with gcc (test infrastructure only)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gqa_oracle.c")
LIB = os.path.join(HERE, "libgqa_oracle.so")


def build(verbose: bool = False) -> str:
    """Always recompile; returns the library path."""
    cmd = ["gcc", "-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
           "-shared", "-fPIC", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
