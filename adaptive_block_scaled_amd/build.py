"""Build libif4.so (HIP for gfx950) in-tree with hipcc.

Flags:
  --offload-arch=gfx950         MI355X only.
  -ffp-contract=off             no implicit fma: every fused multiply-add in
                                the kernels is written explicitly, so the
                                fp32 error sums are exactly the ops stated.
  -fno-gpu-flush-denormals-to-zero, -fhip-fp32-correctly-rounded-divide-sqrt
                                IEEE fp32 (denormals kept, exact division).
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                no packed fp32 (v_pk_*_f32) code generation.

`python -m adaptive_block_scaled_amd.build --sanitize` also builds
libif4_san.so: the host-only C-ABI front end (argument validation) compiled by
the ROCm toolchain's clang++ with AddressSanitizer and UndefinedBehaviorSanitizer,
linked with the same kernel objects.  The binding loads it when IF4_LIB names
it; the sanitizer runtime must be preloaded (the command is in the design doc).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libif4.so")
SAN_LIB = os.path.join(HERE, "libif4_san.so")
CLANGXX = "/opt/rocm/llvm/bin/clang++"

SOURCES = ["api.cpp", "quantize.hip", "dequantize.hip", "gemm.hip", "ifn.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, jobs: int = 4) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC] + COMMON + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    while procs:
        _wait(procs.pop(0))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "--offload-arch=gfx950", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _wait(item):
    src, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    # hipcc's host pass does not know the packed-fp32 target feature; that
    # warning is expected and harmless
    lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
    if p.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError(f"hipcc failed on {src}")
    if any(l.strip() for l in lines):
        sys.stderr.write("\n".join(lines) + "\n")


def build_sanitized_front_end(verbose: bool = False) -> str:
    """api.cpp (host code only) with ASan + UBSan, linked with the kernel
    objects of the last build()."""
    objdir = os.path.join(HERE, "_build")
    kernels = [os.path.join(objdir, s + ".o") for s in SOURCES if s.endswith(".hip")]
    missing = [k for k in kernels if not os.path.exists(k)]
    if missing:
        build(verbose=verbose)
    api_obj = os.path.join(objdir, "api_san.o")
    cmd = [CLANGXX, "-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer",
           "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-c", os.path.join(CSRC, "api.cpp"), "-o", api_obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    cmd = [HIPCC, "-shared", "--offload-arch=gfx950", "-fPIC", "-shared-libsan",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-o", SAN_LIB + ".tmp", api_obj] + kernels
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(SAN_LIB + ".tmp", SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized_front_end(verbose=True))
    else:
        print(build(verbose=True))
