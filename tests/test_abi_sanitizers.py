"""The C ABI's argument checks under AddressSanitizer and UndefinedBehaviorSanitizer.

The host code of every library source is built with both sanitizers (the
device code as usual), and ``abi_sanitize/driver.c`` calls every entry point
with arguments the checks must reject: sizes at the int64 limits, negative
and overflowing strides, unusable windows and mask shapes, problems too large
for a grid or for the allocation-free backward's scratch.  A sanitizer
report aborts the driver; a status other than the documented one fails it.
No call reaches the GPU (every one is rejected first), and the run hides any
GPU from the process all the same.  CPU only; takes about a minute.
"""
import concurrent.futures
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "io_aware_exact_12_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
DRIVER = os.path.join(ROOT, "tests", "abi_sanitize", "driver.c")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="no ROCm compilers")
def test_abi_checks_under_sanitizers(tmp_path):
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))

    def compile_one(f):
        obj = str(tmp_path / (f + ".o"))
        _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN,
              "-I", INCLUDE, "-I", CSRC, "-Wno-unused-command-line-argument",
              "-c", os.path.join(CSRC, f), "-o", obj])
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = str(tmp_path / "libfa_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SAN[:4], "-o", lib, *objs])
    exe = str(tmp_path / "driver")
    _run([CLANG, "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-I", INCLUDE, DRIVER, "-o", exe, "-L", str(tmp_path), "-lfa_san",
          f"-Wl,-rpath,{tmp_path}", "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, f"driver failed ({r.returncode}):\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "all checks passed" in r.stdout
