"""The C ABI layer's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

tests/sanitize/abi_driver.c calls every entry point with NULL, misaligned
and out-of-range arguments, invalid and extreme shapes, and valid
arguments; the layer (csrc/mla_abi.hip, host side only) is built with both
sanitizers and linked with launch stubs (tests/sanitize/abi_stubs.cpp) that
fail every launch, so nothing needs a GPU. The driver exits non-zero on an
unexpected status; the sanitizers abort it on any report.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_abi_layer_under_host_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not (os.path.exists(hipcc) and os.path.exists(CLANG) and os.path.exists(CLANGXX)):
        pytest.skip("ROCm compilers not found")
    # host code only: each sanitizer flag applies to the host pass
    host = ["-std=c++17", "-O1", "-g", "-fPIC", "--cuda-host-only",
            "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-I" + os.path.join(ROOT, "include")]
    _run([hipcc, *host, "-c", os.path.join(ROOT, "latent_kv_attention_amd", "csrc", "mla_abi.hip"), "-o", "abi.o"],
         tmp_path)
    _run([hipcc, *host, "-c", "-x", "hip", os.path.join(SAN, "abi_stubs.cpp"), "-o", "stubs.o"], tmp_path)
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    _run([CLANG, "-O1", "-g", *san, "-c", os.path.join(SAN, "abi_driver.c"), "-o", "driver.o"], tmp_path)
    _run([CLANGXX, *san, "abi.o", "stubs.o", "driver.o", "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", "driver"], tmp_path)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(tmp_path / "driver")], cwd=tmp_path, capture_output=True, text=True, env=env,
                       timeout=120)
    print(r.stdout[-2000:], r.stderr[-2000:])
    assert r.returncode == 0 and "ok: 0 unexpected statuses" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
