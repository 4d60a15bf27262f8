"""Build the IF4 reference oracle (test infrastructure) with gcc.

The oracle is plain C; it is compiled with contraction off and no fast-math
so that every fp32 operation in the error sums is the one written.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build_oracle(verbose: bool = False) -> str:
    src = os.path.join(HERE, "if4_oracle.c")
    cmd = [
        "gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
        "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fno-finite-math-only",
        "-o", LIB + ".tmp", src, "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build_oracle(verbose=True))
