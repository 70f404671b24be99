"""Ahead-of-time build of libmx4.so for gfx950 (hipcc, no JIT, no torch headers).

``python -m microscaled_mxfp4_block_amd.build`` compiles the HIP sources under
``csrc/`` into ``microscaled_mxfp4_block_amd/libmx4.so`` and checks the gfx950
assembly of every kernel source for packed fp32 instructions, which this
build keeps out (``-target-feature -packed-fp32-ops``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmx4.so")
BUILD_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# (source, extra flags, object name): the GEMM is compiled once per K-step budget
SOURCES = [("mx4_api.cpp", [], "mx4_api"), ("mx4_quant.hip", [], "mx4_quant"),
           ("mx4_noalloc.hip", [], "mx4_noalloc"), ("mx4_stream.hip", [], "mx4_stream"),
           ("mx4_shared.hip", [], "mx4_shared"), ("mx4_tile.hip", [], "mx4_tile")] + [
    ("mx4_gemm.hip", ["-DMX4_KR=%d" % kr], "mx4_gemm_kr%d" % kr) for kr in (1, 2, 3, 4, 8)]
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-I" + os.path.join(ROOT, "include")]
# Kernel sources: the first 14 SGPRs of kernel arguments are preloaded at wave
# launch (the GEMM kernels' leading scalar arguments, the quantisers' pointers
# and sizes), so a kernel's first loads do not wait on a scalar-memory round
# trip to the argument segment.
KERNEL_FLAGS = ["-mllvm", "-amdgpu-kernarg-preload-count=14"]
PACKED_FP32 = re.compile(r"\bv_pk_(add|mul|fma|mov)_f32\b")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), out))
    return out


def _flags(src, extra):
    return FLAGS + (KERNEL_FLAGS if src.endswith(".hip") else []) + extra


def _compile(item):
    src, extra, name = item
    obj = os.path.join(BUILD_DIR, name + ".o")
    _run([HIPCC] + _flags(src, extra) + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
    return obj


def _device_asm(item):
    src, extra, name = item
    asm = os.path.join(BUILD_DIR, name + ".s")
    _run([HIPCC] + _flags(src, extra) + ["-x", "hip", "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", asm])
    with open(asm) as f:
        text = f.read()
    bad = sorted(set(m.group(0) for m in PACKED_FP32.finditer(text)))
    if bad:
        raise RuntimeError("%s: packed fp32 instructions in gfx950 code: %s" % (src, ", ".join(bad)))
    return asm


EXT = os.path.join(HERE, "_mx4ext.so")
HWLIB = os.path.join(HERE, "libmx4hw.so")
HWSRC = ("mx4_hwcheck.hip", [], "mx4_hwcheck")


def build_ext():
    """The CPython fast-call module for the hot entry points (gcc, links libmx4.so)."""
    import sysconfig
    inc = sysconfig.get_paths()["include"]
    tmp = EXT + ".tmp%d" % os.getpid()
    _run(["gcc", "-O2", "-shared", "-fPIC", "-Wall", "-I" + inc, os.path.join(CSRC, "mx4_pyext.c"),
          "-o", tmp, "-L" + HERE, "-lmx4", "-Wl,-rpath,$ORIGIN"])
    os.replace(tmp, EXT)


def build(verbose: bool = False) -> str:
    """Compile every source and link libmx4.so (plus the fast-call module and
    the hardware-check library of the tests); returns libmx4.so's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    kernels = [s for s in SOURCES if s[0].endswith(".hip")] + [HWSRC]
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES + [HWSRC]))
        list(ex.map(_device_asm, kernels))
    hw_obj = objs.pop()
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs)
    os.replace(tmp, LIB)
    tmp = HWLIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp, hw_obj])
    os.replace(tmp, HWLIB)
    build_ext()
    if verbose:
        print("built", LIB, "and", EXT)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
