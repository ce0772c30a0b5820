"""MI355X (gfx950) implementation of the Kamera position-free KV reuse operator.

The compute lives in libkamera.so (HIP kernels behind the C ABI of
include/kamera.h); `position_free_kv_amd.abi` is its ctypes binding.
Importing the package does not load the library.
"""
__all__ = ["abi"]
