"""Build the IF4 reference oracle (test infrastructure) with gcc.

The oracle is plain C; it is compiled with contraction off and no fast-math
so that every fp32 operation in the error sums is the one written.

`python -m oracle.build --sanitize` builds liboracle_san.so instead, with
AddressSanitizer and UndefinedBehaviorSanitizer (clang from the ROCm
toolchain, so that it shares one sanitizer runtime with the C-ABI front end
built by `python -m adaptive_block_scaled_amd.build --sanitize`).  Loading
it needs that runtime preloaded; the command is given in the design doc.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
# IF4_ORACLE_LIB selects another build of the same source (the sanitizer build)
LIB = os.environ.get("IF4_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")
SAN_LIB = os.path.join(HERE, "liboracle_san.so")
CLANG = "/opt/rocm/llvm/bin/clang"


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


def build_oracle_sanitized(verbose: bool = False) -> str:
    src = os.path.join(HERE, "if4_oracle.c")
    cmd = [
        CLANG, "-O1", "-g", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-fast-math", "-fno-omit-frame-pointer",
        "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared-libsan",
        "-o", SAN_LIB + ".tmp", src, "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(SAN_LIB + ".tmp", SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    import sys
    if "--sanitize" in sys.argv:
        print(build_oracle_sanitized(verbose=True))
    else:
        print(build_oracle(verbose=True))
