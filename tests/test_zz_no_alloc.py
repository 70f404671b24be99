"""mx_gemm_noalloc (the entry point for callers that cannot allocate) against
mx_gemm on the same inputs: two calls in a row through the C ABI, the second
on a smaller input, each bit-identical to mx_gemm with a caller's workspace
(same plan, same kernels) and within the oracle tolerance."""
import sys

import numpy as np
import pytest
import torch

import oracle
from microscaled_mxfp4_block_amd import binding as B
from microscaled_mxfp4_block_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tol_ok(g_bits, r_bits):
    g = (g_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    r = (r_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    a = np.abs(r)
    e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -126)
    ulp = np.where(a > 0, np.ldexp(1.0, (e - 7).astype(np.int64)), np.ldexp(1.0, -133))
    return bool((np.abs(g - r) <= 2 * ulp + 1e-3 * np.sqrt(np.mean(r * r))).all())


# (M, N, K): the first needs the pre-quantised activation and split-K
# partials in the scratch array, the second (a smaller input) split-K
# partials only
SEQUENCE = [(256, 2112, 7168), (16, 2112, 7168)]


def test_noalloc_matches_mx_gemm_two_calls():
    for M, N, K in SEQUENCE:
        assert B.mx_gemm_workspace_bytes(M, N, K) > 0
    results = []
    for i, (M, N, K) in enumerate(SEQUENCE):
        say("noalloc call", i, (M, N, K), B.mx_gemm_plan(M, N, K))
        A, Bm = inputs.shape_inputs(M, N, K, seed=500 + i)
        Ad, packed = A.to(DEV), B.mx_pack_weight(Bm.to(DEV))
        C_ref = B.mx_gemm(Ad, packed, N)
        C_na = torch.full((M, N), -3.0, dtype=torch.bfloat16, device=DEV)
        B.mx_gemm_noalloc(Ad, packed, N, C=C_na)
        torch.cuda.synchronize()
        g, r = inputs.bits(C_na.cpu()), inputs.bits(C_ref.cpu())
        assert np.array_equal(g, r), "call %d differs from mx_gemm" % i
        assert tol_ok(g, oracle.gemm(inputs.bits(A), inputs.bits(Bm)))
        results.append(g)
    assert len(results) == 2


# two large-M calls that the planner sends to the tile mode (the activation
# pre-quantised into the scratch array), the second on a smaller input
TILE_SEQUENCE = [(1024, 4096, 1024), (896, 4096, 1024)]


def test_noalloc_tile_mode_matches_mx_gemm():
    for M, N, K in TILE_SEQUENCE:
        assert B.mx_gemm_plan(M, N, K)["amode"] == B.MX_AMODE_TILE
        assert 0 < B.mx_gemm_workspace_bytes(M, N, K) <= B.MX_NOALLOC_SCRATCH_BYTES
    for i, (M, N, K) in enumerate(TILE_SEQUENCE):
        say("noalloc tile call", i, (M, N, K), B.mx_gemm_plan(M, N, K))
        A, Bm = inputs.shape_inputs(M, N, K, seed=700 + i)
        Ad, packed = A.to(DEV), B.mx_pack_weight(Bm.to(DEV))
        C_ref = B.mx_gemm(Ad, packed, N)
        C_na = torch.full((M, N), -3.0, dtype=torch.bfloat16, device=DEV)
        B.mx_gemm_noalloc(Ad, packed, N, C=C_na)
        torch.cuda.synchronize()
        g, r = inputs.bits(C_na.cpu()), inputs.bits(C_ref.cpu())
        assert np.array_equal(g, r), "tile call %d differs from mx_gemm" % i
        assert tol_ok(g, oracle.gemm(inputs.bits(A), inputs.bits(Bm)))
