"""Build the plain-C caller of the library (tests/c_abi/rehydrate_demo.c) next to its source.

    python -m tests.c_abi.build_demo

gcc compiles it as C11 against include/kamera.h and links libkamera.so (rpath to the
package directory and ROCm's lib), so the header is also checked to compile as C.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "position_free_kv_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
DEMO = os.path.join(HERE, "rehydrate_demo")


def build() -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}", os.path.join(HERE, "rehydrate_demo.c"),
           f"-L{PKG}", "-lkamera", f"-L{ROCM}/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../position_free_kv_amd", f"-Wl,-rpath,{ROCM}/lib", "-o", DEMO + ".tmp"]
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(DEMO + ".tmp", DEMO)
    return DEMO


if __name__ == "__main__":
    build()
