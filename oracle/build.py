"""Build the CPU oracle shared library (test infrastructure).

Plain single-threaded C++17 with g++, no fused multiply-add contraction, so
every fp64 expression rounds as written.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["oracle_core.cpp", "oracle_draft.cpp", "oracle_verify.cpp", "oracle_schedule.cpp",
           "oracle_train.cpp", "oracle_rnn.cpp"]
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", LIB + ".tmp"] + [os.path.join(HERE, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
