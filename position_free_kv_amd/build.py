"""Build libkamera.so (HIP, gfx950) in-tree with hipcc.

    python -m position_free_kv_amd.build

The library is the C ABI of include/kamera.h: host validation and packing
(csrc/kamera_host.cpp) plus the gfx950 kernels: the operator
(csrc/kamera_kernels.hip), the patch builder (csrc/kamera_builder.hip) and the
streaming probes used for measurement (csrc/kamera_probe.hip).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libkamera.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = os.environ.get("KAMERA_OFFLOAD_ARCH", "gfx950")

# Packed fp32 VALU forms stay disabled: plain fp32 code only. MFMA accumulators stay
# in ordinary VGPRs, so the independent 16x16 tiles of a task issue back to back
# instead of being funnelled through one set of accumulation registers.
HIP_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose_asm: bool = False) -> str:
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    kobj = os.path.join(objdir, "kamera_kernels.o")
    bobj = os.path.join(objdir, "kamera_builder.o")
    hobj = os.path.join(objdir, "kamera_host.o")
    pobj = os.path.join(objdir, "kamera_probe.o")
    _run([cc, f"--offload-arch={ARCH}", *COMMON, *HIP_FLAGS, "-c",
          os.path.join(CSRC, "kamera_kernels.hip"), "-o", kobj])
    _run([cc, f"--offload-arch={ARCH}", *COMMON, *HIP_FLAGS, "-c",
          os.path.join(CSRC, "kamera_builder.hip"), "-o", bobj])
    _run([cc, f"--offload-arch={ARCH}", *COMMON, *HIP_FLAGS, "-c",
          os.path.join(CSRC, "kamera_probe.hip"), "-o", pobj])
    _run([cc, "-x", "c++", *COMMON, "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", "-c",
          os.path.join(CSRC, "kamera_host.cpp"), "-o", hobj])
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", kobj, bobj, pobj, hobj, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose_asm:
        _run([cc, f"--offload-arch={ARCH}", *COMMON, *HIP_FLAGS, "--cuda-device-only", "-S",
              os.path.join(CSRC, "kamera_kernels.hip"), "-o", os.path.join(objdir, "kamera_kernels.s")])
    return LIB


if __name__ == "__main__":
    build(verbose_asm="--asm" in sys.argv)
