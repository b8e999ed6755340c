"""Builds the C oracle (oracle/c/kvz_oracle.c) into oracle/libkvz_oracle.so with gcc.

Test infrastructure only: the library is loaded by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "c", "kvz_oracle.c")
OUT = os.path.join(HERE, "libkvz_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-Wall", SRC, "-o", OUT + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
