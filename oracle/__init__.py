"""CPU oracle for the MXFP4 GEMM path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never loads it and
it shares no code with the HIP path.

The arithmetic lives in ``mxoracle.c`` (plain C, fp64 accumulation); this
module only builds it with gcc when needed and marshals numpy arrays.  The
rule it follows is the MXFP4 quantisation of the kernelindex.com amd-mxfp4-mm
pages (submission 755056, section "Software MXFP4 quant"), the dequantisation
(-1)^sign * e2m1 * 2^(byte-127), and C = bf16_RNE(fp64 sum of products).
``gemm`` quantises both operands; ``gemm_a16w4`` is the pages' a16wfp4
product, which leaves A in bf16 and quantises only B.

Pins (tests marked ``not gpu``): hand-worked groups under ``tests/golden``,
an independent exact pure-Python brute force (``oracle.bruteforce``), closed
forms and invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxoracle.c")
_LIB = os.path.join(_HERE, "libmxoracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile mxoracle.c into libmxoracle.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-Wall",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # MX_ORACLE_LIB names another build of mxoracle.c (the mutation tests
        # load deliberately broken copies this way to show the pins catch them)
        path = os.environ.get("MX_ORACLE_LIB")
        if not path:
            build()
            path = _LIB
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.mxo_quant.argtypes = [P, I, I, I, P, P]
        lib.mxo_quant.restype = I
        lib.mxo_dequant.argtypes = [P, P, I, I, P]
        lib.mxo_dequant.restype = I
        lib.mxo_gemm_dequantised.argtypes = [P, P, I, I, I, P]
        lib.mxo_gemm_dequantised.restype = I
        lib.mxo_e2m1_code.argtypes = [ctypes.c_double]
        lib.mxo_e2m1_code.restype = I
        lib.mxo_scale_byte.argtypes = [ctypes.c_float]
        lib.mxo_scale_byte.restype = I
        lib.mxo_decode.argtypes = [I, I]
        lib.mxo_decode.restype = ctypes.c_double
        lib.mxo_bf16_to_double.argtypes = [P, ctypes.c_longlong, P]
        lib.mxo_bf16_to_double.restype = I
        lib.mxo_bf16_from_double.argtypes = [ctypes.c_double]
        lib.mxo_bf16_from_double.restype = ctypes.c_uint16
        lib.mxo_num_threads.argtypes = []
        lib.mxo_num_threads.restype = I
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def quant(x_bf16: np.ndarray):
    """bf16 bits [rows, K] (uint16) -> (codes [rows, K/2] u8, bytes [rows, K/32] u8)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, K = x.shape
    codes = np.zeros((rows, K // 2), np.uint8)
    scales = np.zeros((rows, K // 32), np.uint8)
    if _load().mxo_quant(_ptr(x), rows, K, K, _ptr(codes), _ptr(scales)) != 0:
        raise ValueError("oracle quant: bad shape %r" % (x.shape,))
    return codes, scales


def dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Packed codes [rows, K/2] + bytes [rows, K/32] -> fp64 [rows, K]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, half = codes.shape
    K = half * 2
    if scales.shape != (rows, K // 32):
        raise ValueError("oracle dequant: scale shape mismatch")
    out = np.zeros((rows, K), np.float64)
    if _load().mxo_dequant(_ptr(codes), _ptr(scales), rows, K, _ptr(out)) != 0:
        raise ValueError("oracle dequant: bad shape")
    return out


def gemm_dequantised(Ad: np.ndarray, Bd: np.ndarray) -> np.ndarray:
    """bf16 bits of RNE(sum_k Ad[m,k] Bd[n,k]) accumulated in fp64."""
    Ad = np.ascontiguousarray(Ad, dtype=np.float64)
    Bd = np.ascontiguousarray(Bd, dtype=np.float64)
    M, K = Ad.shape
    N, K2 = Bd.shape
    if K != K2:
        raise ValueError("oracle gemm: K mismatch")
    C = np.zeros((M, N), np.uint16)
    _load().mxo_gemm_dequantised(_ptr(Ad), _ptr(Bd), M, N, K, _ptr(C))
    return C


def gemm(A_bf16: np.ndarray, B_bf16: np.ndarray) -> np.ndarray:
    """The whole path: quantise A and B, dequantise, fp64 GEMM, bf16 bits [M, N]."""
    ca, sa = quant(A_bf16)
    cb, sb = quant(B_bf16)
    return gemm_dequantised(dequant(ca, sa), dequant(cb, sb))


def bf16_values(x_bf16: np.ndarray) -> np.ndarray:
    """Exact fp64 values of bf16 bits (any shape)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    out = np.zeros(x.shape, np.float64)
    _load().mxo_bf16_to_double(_ptr(x), x.size, _ptr(out))
    return out


def gemm_a16w4(A_bf16: np.ndarray, B_bf16: np.ndarray) -> np.ndarray:
    """The a16wfp4 product (routing notes of submission 733989: bf16 A times
    fp4 B, no activation quantisation): A's bf16 values as they are, B
    quantised and dequantised by the rule above, the fp64 sum rounded once to
    bf16; bits [M, N]."""
    cb, sb = quant(B_bf16)
    return gemm_dequantised(bf16_values(A_bf16), dequant(cb, sb))


def e2m1_code(q: float) -> int:
    return _load().mxo_e2m1_code(float(q))


def scale_byte(amax: float) -> int:
    return _load().mxo_scale_byte(float(amax))


def decode(code: int, byte: int) -> float:
    return _load().mxo_decode(int(code), int(byte))


def bf16_from_double(d: float) -> int:
    return int(_load().mxo_bf16_from_double(float(d)))


def num_threads() -> int:
    return _load().mxo_num_threads()
