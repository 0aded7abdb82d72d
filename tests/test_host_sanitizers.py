"""The library's host code (argument checks, packer, size queries) built with
AddressSanitizer and UndefinedBehaviorSanitizer on the host side only, and
driven by tests/host/abi_driver.cpp: no GPU is touched (device pointers are
fake addresses the library only inspects).  The device code of the other
objects is linked unchanged; the driver calls nothing that launches it."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "memory_bound_quantized_amd", "_build")
CSRC = os.path.join(ROOT, "memory_bound_quantized_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"


def test_host_code_under_asan_and_ubsan():
    objs = [os.path.join(BUILD, f) for f in sorted(os.listdir(BUILD))
            if f.endswith(".o") and f != "abi.o"] if os.path.isdir(BUILD) else []
    if not objs or not os.path.exists(HIPCC) or not os.path.exists(CLANG):
        pytest.skip("needs the built objects (build()) and the ROCm compilers")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    with tempfile.TemporaryDirectory() as tmp:
        abi_o, drv_o, exe = (os.path.join(tmp, n) for n in ("abi_san.o", "driver.o", "abi_driver"))
        subprocess.run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + san +
                       ["-I" + os.path.join(ROOT, "include"), "-x", "hip", "-c",
                        os.path.join(CSRC, "abi.cpp"), "-o", abi_o],
                       check=True, capture_output=True)
        host = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer"]
        subprocess.run([CLANG, "-O1", "-g", "-std=c++17"] + host +
                       ["-I" + os.path.join(ROOT, "include"), "-c",
                        os.path.join(ROOT, "tests", "host", "abi_driver.cpp"), "-o", drv_o],
                       check=True, capture_output=True)
        subprocess.run([CLANG] + host + ["-o", exe, drv_o, abi_o] + objs +
                       ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"],
                       check=True, capture_output=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
