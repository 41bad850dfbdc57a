"""Host-sanitized build of the library, for the CPU checks of the C-ABI's host logic.

sf_host.cpp (the C-ABI: argument checks, slot bookkeeping, launch planning, state
export/import) is compiled with AddressSanitizer and UndefinedBehaviorSanitizer on the host
side only (every sanitizer flag goes through -Xarch_host; the gfx950 device code is built as
usual).  The result, _build/libsf_asan.so, is linked into a sanitized C driver by
tests/test_host_sanitized.py; the Python package never loads it.

Usage: python compressed_memory_kv_amd/build_sanitized.py
"""
from __future__ import annotations

import importlib.util
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
OUT = os.path.join(ROOT, "_build", "libsf_asan.so")

_spec = importlib.util.spec_from_file_location("sf_build", os.path.join(HERE, "build.py"))
_b = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(_b)

HOST_SANITIZE = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-g",
]
LINK_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"]


def build(verbose: bool = False) -> str:
    return _b.build(verbose=verbose, out=OUT, file_flags={"sf_host.cpp": HOST_SANITIZE}, link_flags=LINK_SANITIZE)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
