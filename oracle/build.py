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


def build(verbose: bool = False, out: str = OUT, sanitize: bool = False) -> str:
    """sanitize: AddressSanitizer and UndefinedBehaviorSanitizer (every report fatal), for the
    CPU test that runs the oracle's pins under them; the process that loads such a library must
    preload libasan (sanitizer_runtime())."""
    opt = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined"] if sanitize else ["-O2"]
    cmd = ["gcc", *opt, "-fPIC", "-shared", "-fopenmp", "-std=c11", "-Wall", SRC, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def sanitizer_runtime() -> str:
    """Path of gcc's AddressSanitizer runtime, to preload into a process that loads a sanitized
    oracle."""
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
