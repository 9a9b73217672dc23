"""The host-side argument checks of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer: abi.cpp is rebuilt with host-only sanitizers
(the device code is untouched), linked with the normally built kernel
objects, and tests/test_abi_cpu.py runs against that library in a child
process with the sanitizer runtime preloaded.  Any report fails the run.
CPU only (the checks run before any HIP call)."""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.skipif(not os.path.exists(HIPCC) or _asan_runtime() is None, reason="hipcc or its ASan runtime missing")
def test_abi_checks_under_asan_ubsan(tmp_path):
    objs = [o for o in glob.glob(os.path.join(BUILD, "*.o")) if not os.path.basename(o).startswith("abi.cpp")]
    if not objs:
        pytest.skip("the library has not been built (no kernel objects in _build)")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    abi_o = str(tmp_path / "abi_san.o")
    lib = str(tmp_path / "libmoe_san.so")
    cmd = [HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-x", "hip",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), *san,
           "-c", os.path.join(ROOT, "bit_quantized_expert_amd", "csrc", "abi.cpp"), "-o", abi_o]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", "-o", lib, abi_o, *objs], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), MOE_ABI_TEST_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert "passed" in out
