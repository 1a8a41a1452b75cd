"""Compile the seeded input generator (synth.c) into synth/libsynth.so with gcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libsynth.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "synth.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fno-fast-math", "-pthread", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
