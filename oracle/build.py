"""Build the fp64 CPU oracle (test infrastructure) into oracle/libstreamkl_oracle.so.

Plain gcc, strict IEEE (no -ffast-math), OpenMP across rows.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "streamkl_oracle.c")
LIB = os.path.join(HERE, "libstreamkl_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
