"""libif4: IF4 (Int/Float 4) adaptive block-scaled quantization for MI355X.

The compute path is the HIP library libif4.so (C ABI in include/if4.h); the
Python side in `if4` only marshals pointers, sizes and the stream.  Import
of this package is cheap: the library is loaded on first use.
"""
__all__ = ["if4", "workloads"]
