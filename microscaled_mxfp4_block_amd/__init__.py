"""MI355X-native MXFP4 GEMM: C[M,N] (bf16) = A[M,K] x B[N,K]^T with on-the-fly
activation quantisation, behind the C ABI declared in include/mx4.h.

The Python names mirror the C entry points (see ``binding``); the HIP library
``libmx4.so`` must be built first (``python -m microscaled_mxfp4_block_amd.build``).
"""
from .binding import (  # noqa: F401
    MxError,
    mx_gemm,
    mx_gemm_a16w4,
    mx_gemm_plan,
    mx_gemm_workspace_bytes,
    mx_import_weight,
    mx_pack_weight,
    mx_packed_weight_bytes,
    mx_quant_act,
    mx_unpack_weight,
    strerror,
)
