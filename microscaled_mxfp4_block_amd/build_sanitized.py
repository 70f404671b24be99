"""Host-sanitizer build of the library for CPU tests (never run on a GPU).

``python -m microscaled_mxfp4_block_amd.build_sanitized`` compiles the same
sources as ``build.py`` with the host code (argument validation, planner,
workspace layout, the prepared-call cache, the C ABI) under AddressSanitizer
and UndefinedBehaviorSanitizer, and links ``_build/asan/libmx4.so``.  Device
code is built as usual (no GPU sanitizer).  ``tests/test_abi_sanitized.py``
runs the C-ABI tests against it, with the ASan runtime preloaded.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

from . import build as B

OUT_DIR = os.path.join(B.BUILD_DIR, "asan")
LIB = os.path.join(OUT_DIR, "libmx4.so")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def asan_runtime() -> str:
    """Path of the clang ASan runtime the sanitized library needs preloaded."""
    out = subprocess.run([B.HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE,
                         text=True, check=True).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        import glob
        cands = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
        if not cands:
            raise RuntimeError("clang ASan runtime not found")
        out = cands[-1]
    return out


def _compile(item):
    src, extra, name = item
    obj = os.path.join(OUT_DIR, name + ".o")
    B._run([B.HIPCC] + B._flags(src, extra) + HOST_SAN + ["-x", "hip", "-c", os.path.join(B.CSRC, src), "-o", obj])
    return obj


def build() -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, B.SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    B._run([B.HIPCC, "-shared", "-fPIC", "--offload-arch=" + B.ARCH, "-shared-libsan", "-Xarch_host",
            "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)
