"""The C-ABI's host logic under AddressSanitizer, UndefinedBehaviorSanitizer and
LeakSanitizer (CPU only, no GPU needed).

compressed_memory_kv_amd/build_sanitized.py builds the library with the sanitizers on the
host side only; tests/sanitize/host_api_check.c, built with the same sanitizers, drives
every entry point on dry-run handles (the served, long-horizon and small shapes, every rope
mode, the sink, the recency bias, the zero-copy slot, batched reads, state export/import
and corrupted state, and the error paths).  Any sanitizer finding aborts the driver.
"""
import glob
import importlib.util
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


def _runtime_dir():
    libs = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return os.path.dirname(libs[0]) if libs else None


HAVE_TOOLS = os.path.exists(CLANG) and (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc"))


@pytest.mark.skipif(not HAVE_TOOLS or _runtime_dir() is None, reason="needs the ROCm toolchain and its sanitizer runtimes")
def test_host_api_under_sanitizers():
    spec = importlib.util.spec_from_file_location(
        "sf_build_sanitized", os.path.join(ROOT, "compressed_memory_kv_amd", "build_sanitized.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    lib = mod.build()
    exe = os.path.join(os.path.dirname(lib), "host_api_check")
    rt = _runtime_dir()
    cmd = [CLANG, "-std=c11", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-shared-libsan", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "sanitize", "host_api_check.c"), "-L", os.path.dirname(lib), "-lsf_asan",
           f"-Wl,-rpath,{os.path.dirname(lib)}", f"-Wl,-rpath,{rt}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "host API checks passed" in out
    assert "runtime error" not in out and "AddressSanitizer" not in out and "LeakSanitizer" not in out, out[-4000:]
