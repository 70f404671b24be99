"""Thin ctypes binding of libmx4.so (include/mx4.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
the library.  PyTorch supplies device memory and the current stream.  If the
library has not been built, the first call raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MX4_LIBRARY names another build of the same library (the host-sanitizer
# build of the CPU tests); by default the one built next to this file.
LIB_PATH = os.environ.get("MX4_LIBRARY") or os.path.join(_HERE, "libmx4.so")

MX_OK = 0
MX_EINVAL = -1
MX_EALIGN = -2
MX_ESPACE = -3
MX_EHIP = -4
MX_EPLAN = -5
# activation modes of a plan (where A is quantised)
MX_AMODE_LDS = 0
MX_AMODE_PREQUANT = 1
MX_AMODE_DIRECT = 2
MX_AMODE_BF16 = 3          # A not quantised: the a16wfp4 product
MX_AMODE_STREAM = 4        # per-wave quantisation in a K loop
MX_AMODE_SHARED = 5        # quantiser waves into LDS for MFMA waves
MX_AMODE_TILE = 6          # pre-quantised A, K-looped LDS-tiled GEMM (M from 64)
# split-K finishes of a plan
MX_FINISH_KERNEL = 0
MX_FINISH_LAST_ARRIVAL = 1

EXPORTS = [
    "mx_strerror", "mx_packed_weight_bytes", "mx_pack_weight", "mx_unpack_weight",
    "mx_import_weight", "mx_quant_act", "mx_gemm_workspace_bytes", "mx_gemm", "mx_gemm_plan",
    "mx_gemm_plan_workspace_bytes", "mx_gemm_with_plan",
    "mx_gemm_a16w4_plan", "mx_gemm_a16w4_workspace_bytes", "mx_gemm_a16w4", "mx_gemm_noalloc",
]
# bytes of the static device workspace of mx_gemm_noalloc (MX_NOALLOC_SCRATCH_BYTES)
MX_NOALLOC_SCRATCH_BYTES = 8 << 20


class MxPlan(ctypes.Structure):
    _fields_ = [("mb", ctypes.c_int), ("nb", ctypes.c_int), ("wn", ctypes.c_int), ("wk", ctypes.c_int),
                ("splits", ctypes.c_int), ("amode", ctypes.c_int),
                ("finish", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class MxError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__("%s failed: %s (%d)" % (where, strerror(code), code))
        self.code = code


_lib = None
_ext = None


def ext():
    """The CPython fast-call module (_mx4ext) for mx_gemm / mx_gemm_with_plan."""
    global _ext
    if _ext is None:
        lib()   # fails loudly when libmx4.so is missing
        from . import _mx4ext
        _ext = _mx4ext
    return _ext


def lib() -> ctypes.CDLL:
    """Load libmx4.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libmx4.so is not built; run `python -m microscaled_mxfp4_block_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        I, P, S = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        PS = ctypes.POINTER(ctypes.c_size_t)
        PP = ctypes.POINTER(MxPlan)
        L.mx_strerror.argtypes = [I]
        L.mx_strerror.restype = ctypes.c_char_p
        L.mx_packed_weight_bytes.argtypes = [I, I, PS]
        L.mx_pack_weight.argtypes = [P, I, I, I, P, S, P]
        L.mx_unpack_weight.argtypes = [P, I, I, P, P, P]
        L.mx_import_weight.argtypes = [P, P, I, I, P, S, P]
        L.mx_quant_act.argtypes = [P, I, I, I, P, P, P]
        L.mx_gemm_workspace_bytes.argtypes = [I, I, I, PS]
        L.mx_gemm.argtypes = [P, I, I, I, P, I, P, I, P, S, P]
        L.mx_gemm_plan.argtypes = [I, I, I, PP]
        L.mx_gemm_plan_workspace_bytes.argtypes = [PP, I, I, I, PS]
        L.mx_gemm_with_plan.argtypes = [P, I, I, I, P, I, P, I, P, S, PP, P]
        L.mx_gemm_a16w4_plan.argtypes = [I, I, I, PP]
        L.mx_gemm_a16w4_workspace_bytes.argtypes = [I, I, I, PS]
        L.mx_gemm_a16w4.argtypes = [P, I, I, I, P, I, P, I, P, S, P]
        L.mx_gemm_noalloc.argtypes = [P, I, I, I, P, I, P, I, P]
        for name in EXPORTS[1:]:
            getattr(L, name).restype = I
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().mx_strerror(code).decode()


def _check(rc: int, where: str):
    if rc != MX_OK:
        raise MxError(rc, where)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _bf16_matrix(t: torch.Tensor, name: str):
    if t.dtype != torch.bfloat16 or t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("%s must be a 2-D bf16 tensor with unit column stride" % name)
    return t.shape[0], t.shape[1], t.stride(0)


def mx_packed_weight_bytes(N: int, K: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().mx_packed_weight_bytes(N, K, ctypes.byref(out)), "mx_packed_weight_bytes")
    return out.value


def mx_pack_weight(B: torch.Tensor, packed: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Pack a bf16 weight [N, K] once; returns the opaque uint8 packed buffer."""
    N, K, ldb = _bf16_matrix(B, "B")
    nbytes = mx_packed_weight_bytes(N, K)
    if packed is None:
        packed = torch.empty(nbytes, dtype=torch.uint8, device=B.device)
    _check(lib().mx_pack_weight(_ptr(B), N, K, ldb, _ptr(packed), packed.numel(), _stream(stream)),
           "mx_pack_weight")
    return packed


def mx_unpack_weight(packed: torch.Tensor, N: int, K: int, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Natural-layout codes [N, K/2] and e8m0 bytes [N, K/32] of a packed weight."""
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=packed.device)
    scales = torch.empty((N, K // 32), dtype=torch.uint8, device=packed.device)
    _check(lib().mx_unpack_weight(_ptr(packed), N, K, _ptr(codes), _ptr(scales), _stream(stream)),
           "mx_unpack_weight")
    return codes, scales


def mx_import_weight(codes: torch.Tensor, scales: torch.Tensor, N: int, K: int, packed: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """Packed weight from natural-layout codes [N, K/2] and e8m0 bytes [N, K/32] quantised elsewhere."""
    for t, name, cols in ((codes, "codes", K // 2), (scales, "scales", K // 32)):
        if t.dtype != torch.uint8 or tuple(t.shape) != (N, cols) or not t.is_contiguous():
            raise ValueError("%s must be a contiguous uint8 [%d, %d] tensor" % (name, N, cols))
    nbytes = mx_packed_weight_bytes(N, K)
    if packed is None:
        packed = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    _check(lib().mx_import_weight(_ptr(codes), _ptr(scales), N, K, _ptr(packed), packed.numel(), _stream(stream)),
           "mx_import_weight")
    return packed


def mx_quant_act(A: torch.Tensor, codes: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
                 stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Quantise bf16 activations [M, K] to natural codes [M, K/2] and e8m0 bytes [M, K/32]."""
    M, K, lda = _bf16_matrix(A, "A")
    if codes is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=A.device)
    if scales is None:
        scales = torch.empty((M, K // 32), dtype=torch.uint8, device=A.device)
    _check(lib().mx_quant_act(_ptr(A), M, K, lda, _ptr(codes), _ptr(scales), _stream(stream)), "mx_quant_act")
    return codes, scales


def mx_gemm_plan(M: int, N: int, K: int) -> dict:
    p = MxPlan()
    _check(lib().mx_gemm_plan(M, N, K, ctypes.byref(p)), "mx_gemm_plan")
    return p.as_dict()


def mx_gemm_workspace_bytes(M: int, N: int, K: int, plan: Optional[dict] = None) -> int:
    out = ctypes.c_size_t(0)
    if plan is None:
        _check(lib().mx_gemm_workspace_bytes(M, N, K, ctypes.byref(out)), "mx_gemm_workspace_bytes")
    else:
        p = MxPlan(**plan)
        _check(lib().mx_gemm_plan_workspace_bytes(ctypes.byref(p), M, N, K, ctypes.byref(out)),
               "mx_gemm_plan_workspace_bytes")
    return out.value


def new_workspace(M: int, N: int, K: int, plan: Optional[dict] = None, device="cuda") -> torch.Tensor:
    """A zero-filled workspace for mx_gemm on this shape (and plan); calls keep its counters zero."""
    nbytes = mx_gemm_workspace_bytes(M, N, K, plan)
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)


def mx_gemm(A: torch.Tensor, packed: torch.Tensor, N: int, C: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None, plan: Optional[dict] = None, stream=None) -> torch.Tensor:
    """C[M, N] (bf16) = A x B^T with A quantised on the fly and B packed by mx_pack_weight."""
    M, K, lda = _bf16_matrix(A, "A")
    if C is None:
        C = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    Mc, Nc, ldc = _bf16_matrix(C, "C")
    if (Mc, Nc) != (M, N):
        raise ValueError("C must be [%d, %d]" % (M, N))
    if workspace is None:
        workspace = new_workspace(M, N, K, plan, device=A.device)
    s = _stream(stream)
    if plan is None:
        rc = ext().gemm(A.data_ptr(), M, K, lda, packed.data_ptr(), N, C.data_ptr(), ldc, workspace.data_ptr(),
                        workspace.numel(), s)
    else:
        rc = ext().gemm_with_plan(A.data_ptr(), M, K, lda, packed.data_ptr(), N, C.data_ptr(), ldc,
                                  workspace.data_ptr(), workspace.numel(), plan["mb"], plan["nb"], plan["wn"],
                                  plan["wk"], plan["splits"], plan["amode"],
                                  plan.get("finish", MX_FINISH_KERNEL), s)
    _check(rc, "mx_gemm")
    return C


def mx_gemm_a16w4_plan(M: int, N: int, K: int) -> dict:
    p = MxPlan()
    _check(lib().mx_gemm_a16w4_plan(M, N, K, ctypes.byref(p)), "mx_gemm_a16w4_plan")
    return p.as_dict()


def mx_gemm_a16w4_workspace_bytes(M: int, N: int, K: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().mx_gemm_a16w4_workspace_bytes(M, N, K, ctypes.byref(out)), "mx_gemm_a16w4_workspace_bytes")
    return out.value


def mx_gemm_a16w4(A: torch.Tensor, packed: torch.Tensor, N: int, C: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """C[M, N] (bf16) = A x dequant(B)^T with A left in bf16 (the a16wfp4 product)."""
    M, K, lda = _bf16_matrix(A, "A")
    if C is None:
        C = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    Mc, Nc, ldc = _bf16_matrix(C, "C")
    if (Mc, Nc) != (M, N):
        raise ValueError("C must be [%d, %d]" % (M, N))
    if workspace is None:
        workspace = torch.zeros(max(mx_gemm_a16w4_workspace_bytes(M, N, K), 256), dtype=torch.uint8,
                                device=A.device)
    rc = ext().gemm_a16w4(A.data_ptr(), M, K, lda, packed.data_ptr(), N, C.data_ptr(), ldc, workspace.data_ptr(),
                          workspace.numel(), _stream(stream))
    _check(rc, "mx_gemm_a16w4")
    return C


def mx_gemm_noalloc(A: torch.Tensor, packed: torch.Tensor, N: int, C: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """mx_gemm with the library's static per-GPU workspace instead of a caller's
    (for callers that cannot allocate); calls on one GPU must not overlap."""
    M, K, lda = _bf16_matrix(A, "A")
    if C is None:
        C = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    Mc, Nc, ldc = _bf16_matrix(C, "C")
    if (Mc, Nc) != (M, N):
        raise ValueError("C must be [%d, %d]" % (M, N))
    _check(lib().mx_gemm_noalloc(A.data_ptr(), M, K, lda, packed.data_ptr(), N, C.data_ptr(), ldc,
                                 _stream(stream)), "mx_gemm_noalloc")
    return C
