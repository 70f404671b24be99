"""The shape grid of the kernelindex.com amd-mxfp4-mm pages (submission
754569, the synthesized config CSV: 19 (N, K) weight shapes times the batch
sizes M = 1, 2, 4, ..., 256, 171 shapes) through mx_gemm with the library's
own plan, against the CPU oracle (needs an MI355X).

Every shape is checked on a sampled sub-grid of C: up to 8 rows (the first,
the last and random ones) by 72 columns (the first 4, the last 4 and 64
random ones), every element of it against the oracle's product of exactly
those rows of A and columns of B (C[m, n] depends only on row m of A and row
n of B), within |C - C_ref| <= 2 ulp_bf16(|C_ref|) + 1e-3 rms(C_ref), the
rms taken over the sampled elements.  Inputs: N(0, 1) bf16 from a per-shape
seed; each weight is drawn and packed once for its nine batch sizes.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from microscaled_mxfp4_block_amd import binding as B
from microscaled_mxfp4_block_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (N, K) pairs and batch sizes of the pages' shape grid
DIM_PAIRS = [
    (2880, 512), (2112, 7168), (4096, 512), (7168, 2048), (3072, 1536),
    (2880, 1536), (4096, 1536), (2112, 512), (2112, 2048),
    (7168, 512), (7168, 1536), (7168, 7168), (3072, 512),
    (3072, 7168), (3072, 2048), (4096, 2048), (4096, 7168),
    (2880, 2048), (2880, 7168),
]
BATCH = [1, 2, 4, 8, 16, 32, 64, 128, 256]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def close(g_bits, r_bits):
    g = (g_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    r = (r_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    a = np.abs(r)
    e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -126)
    ulp = np.where(a > 0, np.ldexp(1.0, (e - 7).astype(np.int64)), np.ldexp(1.0, -133))
    tol = 2 * ulp + 1e-3 * np.sqrt(np.mean(r * r))
    bad = np.abs(g - r) > tol
    return np.isfinite(g).all() and not bad.any(), int(bad.sum())


@pytest.mark.parametrize("nk", DIM_PAIRS, ids=lambda p: "n%d_k%d" % p)
def test_grid_shapes_against_oracle(nk):
    N, K = nk
    gen = torch.Generator("cpu").manual_seed(5000 + N + K)
    Bm = inputs.bf16_randn(N, K, gen)
    packed = B.mx_pack_weight(Bm.to(DEV))
    B_bits = inputs.bits(Bm)
    rng = np.random.default_rng(N * 7 + K)
    cols = np.unique(np.concatenate([np.arange(4), np.arange(N - 4, N), rng.integers(0, N, 64)]))
    for M in BATCH:
        A = inputs.bf16_randn(M, K, gen)
        say("grid", (M, N, K), B.mx_gemm_plan(M, N, K))
        C = B.mx_gemm(A.to(DEV), packed, N)
        got = inputs.bits(C.cpu())
        rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 6)]))
        A_bits = inputs.bits(A)
        ref = oracle.gemm(np.ascontiguousarray(A_bits[rows]), np.ascontiguousarray(B_bits[cols]))
        ok, nbad = close(got[np.ix_(rows, cols)], ref)
        assert ok, "(%d, %d, %d): %d sampled outputs outside tolerance" % (M, N, K, nbad)
