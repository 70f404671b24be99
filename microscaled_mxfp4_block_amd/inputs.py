"""Seeded synthetic inputs for the MXFP4 GEMM workloads.

This module only draws random numbers; it holds none of the quantisation or
GEMM arithmetic.  Both the HIP path (tests, benchmark) and the CPU oracle are
fed from here, so they see identical bf16 bits.

Recipe: for workload ``i`` and a base seed (1000, 2000 or 3000),
``g = torch.Generator("cpu").manual_seed(base + i)``; ``A = randn(M, K)``
then ``B = randn(N, K)`` are drawn in fp32 from ``g`` and rounded (RNE) to
bf16.  The shapes are the decode-style MI355X shapes of the kernelindex.com
amd-mxfp4-mm leaderboard pages (plan tables of submissions 748756 and
754569): the leaderboard's own data generator is not available, so N(0, 1)
inputs of the same shapes stand in for it.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int


# (M, N, K) of the five measured workloads, in a fixed order.
WORKLOADS = [
    Workload("m4_n2880_k512", 4, 2880, 512),
    Workload("m32_n4096_k512", 32, 4096, 512),
    Workload("m16_n2112_k7168", 16, 2112, 7168),
    Workload("m64_n7168_k2048", 64, 7168, 2048),
    Workload("m256_n3072_k1536", 256, 3072, 1536),
]

# A sixth decode shape the same workload family lists (K=512, M=32); inputs
# come from shape_inputs with a per-shape seed.
EXTRA_WORKLOADS = [
    Workload("m32_n2880_k512", 32, 2880, 512),
]


def bf16_randn(rows: int, cols: int, gen: torch.Generator, scale: float = 1.0) -> torch.Tensor:
    """N(0, scale^2) drawn in fp32 from ``gen`` and rounded to a CPU bf16 tensor."""
    x = torch.randn(rows, cols, generator=gen, dtype=torch.float32)
    if scale != 1.0:
        x = x * scale
    return x.to(torch.bfloat16)


def workload_inputs(index: int, base_seed: int = 1000):
    """(A, B) CPU bf16 tensors for workload ``index`` under one base seed."""
    w = WORKLOADS[index]
    g = torch.Generator("cpu").manual_seed(base_seed + index)
    A = bf16_randn(w.M, w.K, g)
    B = bf16_randn(w.N, w.K, g)
    return A, B


def shape_inputs(M: int, N: int, K: int, seed: int, scale_a: float = 1.0, scale_b: float = 1.0):
    """(A, B) CPU bf16 tensors of an arbitrary shape from one seed."""
    g = torch.Generator("cpu").manual_seed(seed)
    return bf16_randn(M, K, g, scale_a), bf16_randn(N, K, g, scale_b)


def binade_spread(rows: int, cols: int, seed: int, lo: int = -20, hi: int = 20) -> torch.Tensor:
    """bf16 matrix whose 32-element groups each sit at a random binade in
    [lo, hi): N(0,1) times 2^e with one e per group, so scales vary widely."""
    g = torch.Generator("cpu").manual_seed(seed)
    x = torch.randn(rows, cols, generator=g, dtype=torch.float32)
    e = torch.randint(lo, hi, (rows, (cols + 31) // 32), generator=g)
    mult = torch.pow(2.0, e.to(torch.float32)).repeat_interleave(32, dim=1)[:, :cols]
    return (x * mult).to(torch.bfloat16)


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (CPU copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(b: np.ndarray) -> torch.Tensor:
    """numpy uint16 bit patterns -> CPU bf16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
