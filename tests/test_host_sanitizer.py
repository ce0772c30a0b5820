"""The library's host code under AddressSanitizer (CPU only).

The host part (argument validation, batch packing, the staging ring) is rebuilt with
g++ -fsanitize=address and linked with the same gfx950 kernel objects; the C-ABI
validation tests (tests/test_abi_cpu.py) then run against that build in a child process
with the ASan runtime preloaded, so every error path walks through instrumented code.
Any sanitizer report fails the test. Device code is not instrumented.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "position_free_kv_amd", "csrc")
OBJS = os.path.join(ROOT, "position_free_kv_amd", "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _gpu_present() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:  # noqa: BLE001
        return False


@pytest.mark.skipif(_gpu_present(), reason="the validation tests it drives use fake device addresses")
def test_host_code_under_address_sanitizer():
    kobjs = [os.path.join(OBJS, f) for f in ("kamera_kernels.o", "kamera_builder.o", "kamera_probe.o")]
    assert all(os.path.exists(o) for o in kobjs), "kernel objects missing: build the library first"
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    assert os.path.isabs(libasan), "no ASan runtime"
    with tempfile.TemporaryDirectory() as d:
        host = os.path.join(d, "host_asan.o")
        lib = os.path.join(d, "libkamera_asan.so")
        cc = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-fsanitize=address", "-fno-omit-frame-pointer",
              "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
              "-c", os.path.join(CSRC, "kamera_host.cpp"), "-o", host]
        subprocess.run(cc, check=True)
        subprocess.run(["g++", "-shared", "-fPIC", *kobjs, host, "-fsanitize=address", f"-L{ROCM}/lib", "-lamdhip64",
                        f"-Wl,-rpath,{ROCM}/lib", "-o", lib], check=True)
        env = dict(os.environ, LD_PRELOAD=libasan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   KAMERA_LIBRARY=lib, PYTHONPATH=ROOT)
        probe = subprocess.run([sys.executable, "-c", "from position_free_kv_amd import abi; abi.lib(); print(abi.LIB_PATH)"],
                               env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
        assert probe.returncode == 0 and probe.stdout.strip() == lib, probe.stderr[-2000:]
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                           env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
        out = r.stdout + r.stderr
        assert r.returncode == 0 and "AddressSanitizer" not in out, out[-3000:]
        assert " passed" in out
