"""Build the plain-C HQMQ oracle (test infrastructure only).

    python oracle/build.py

produces ``oracle/libhqmq_oracle.so`` with gcc.  ``-ffp-contract=off`` keeps
every fp32 operation of the declared norm code rounded on its own.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "hqmq_oracle.c")
LIB = os.path.join(HERE, "libhqmq_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math",
        "-fopenmp", "-shared", "-fPIC", "-Wall", "-Wextra",
        SRC, "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
