"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with both sanitizers on its host code only (the device
code is compiled unoptimized and never launched) and linked into a C driver
(tests/abi_driver.c) that calls every entry point with arguments its
validation must refuse, plus the size queries; no GPU is needed. Any invalid
read or write, overflow or other undefined behaviour in the argument checks,
planning or status paths aborts the driver. The build is cached under
_build/sanitized by a digest of the sources.
"""

import glob
import hashlib
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lora_fine_tuning_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "sanitized")


def _tools():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    clang = "/opt/rocm/llvm/bin/clang"
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not (os.path.exists(hipcc) and os.path.exists(clang) and rt):
        pytest.skip("hipcc, clang or the clang sanitizer runtime is not installed")
    return hipcc, clang, os.path.dirname(rt[0])


def _digest():
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.hpp")))
    files += [os.path.join(ROOT, "include", "lora4.h"), os.path.join(ROOT, "tests", "abi_driver.c")]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _build(hipcc, clang):
    d = os.path.join(OUT, _digest())
    drv = os.path.join(d, "abi_driver")
    if os.path.exists(drv):
        return d, drv
    os.makedirs(d, exist_ok=True)
    lib = os.path.join(d, "liblora4_sanitized.so")
    # sanitizers on the host code only (each -fsanitize= behind -Xarch_host)
    cmd = [hipcc, "--offload-arch=gfx950", "-O0", "-g0", "-std=c++17", "-fPIC", "-shared",
           "-Xarch_host", "-O1", "-Xarch_host", "-g",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libsan",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, "lora4.hip"), "-o", lib]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    cmd = [clang, "-O1", "-g", "-fsanitize=address,undefined", "-shared-libsan", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_driver.c"),
           "-L", d, "-llora4_sanitized", "-Wl,-rpath," + d, "-o", drv]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    return d, drv


def test_abi_host_code_is_clean_under_asan_and_ubsan():
    hipcc, clang, rt = _tools()
    d, drv = _build(hipcc, clang)
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = rt + (":" + env["LD_LIBRARY_PATH"] if env.get("LD_LIBRARY_PATH") else "")
    # the HIP runtime keeps process-lifetime allocations: leak reports are off
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["HIP_VISIBLE_DEVICES"] = ""
    res = subprocess.run([drv], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0 and res.stdout.strip().endswith("ok"), res.stdout[-3000:] + res.stderr[-3000:]
