"""Bit-exact check of the activation quantisers that run inside the GEMM.

The GEMM's own quantisation of A (in registers per wave, into LDS per
workgroup, or by the per-call pre-quantisation kernel) never leaves the
kernel, so it is read out through C: with a weight whose rows are unit
vectors, B[n, k] = 1 when k == (n + off) mod K, every group of B is either
all zero (scale byte 0, zero codes) or holds one 1.0 (amax 1, scale byte
125, code 6 = 4 * 2^-2), so deq(B) is exactly that 0/1 matrix.  Then each
output is a single product, C[m, n] = deq(A)[m, (n + off) mod K], and a
dequantised MXFP4 value (at most two significant bits times a power of two
from 2^-128 up) is exact in fp32 and in bf16.  C must therefore equal the
oracle's dequant(quant(A)) bit for bit, up to the sign of zero (a -0 code
adds into a +0 accumulator and cannot show in C).  That pins every nonzero
code and every scale byte of a group with a nonzero element, for each
activation mode, K split and split-K finish.
"""
import json
import os
import struct
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


def hand_group_rows(M: int, K: int) -> np.ndarray:
    """M x K bf16 bits: the hand-worked groups of tests/golden, tiled along K,
    each row starting at another group, odd rows with every sign flipped."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "hand_groups.json")) as f:
        gs = json.load(f)["groups"]
    groups = np.zeros((len(gs), 32), np.uint16)
    for gi, g in enumerate(gs):
        for k, v in g["values"].items():
            groups[gi, int(k)] = struct.unpack("<I", struct.pack("<f", v))[0] >> 16
    out = np.zeros((M, K), np.uint16)
    for r in range(M):
        for g in range(K // 32):
            out[r, 32 * g:32 * g + 32] = groups[(r + g) % len(gs)]
        if r % 2:
            out[r] ^= 0x8000
    return out


def adversarial(M: int, K: int, seed: int) -> np.ndarray:
    """Hand-worked rows and rows whose groups sit at random binades from
    2^-140 (bf16 subnormals and zeros) to 2^123, interleaved; every
    dequantised value stays below 2^127, inside fp32."""
    hand = hand_group_rows(M, K)
    spread = inputs.bits(inputs.binade_spread(M, K, seed=seed, lo=-140, hi=124))
    out = spread.copy()
    out[0::3] = hand[0::3]
    return out


def unit_weight(N: int, K: int, off: int) -> torch.Tensor:
    """B[n, k] = 1 when k == (n + off) mod K, else 0 (CPU bf16)."""
    Bm = torch.zeros((N, K), dtype=torch.bfloat16)
    n = torch.arange(N)
    Bm[n, (n + off) % K] = 1.0
    return Bm


def expected_deq_bits(A_bits: np.ndarray) -> np.ndarray:
    """bf16 bits of the oracle's dequant(quant(A)); asserts they are exact."""
    d = oracle.dequant(*oracle.quant(A_bits))
    assert np.abs(d).max() < 2.0 ** 127
    f = d.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), d), "dequantised value not exact in fp32"
    u = f.view(np.uint32)
    assert not (u & 0xFFFF).any(), "dequantised value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_extraction(A_bits: np.ndarray, N: int, plan, what: str):
    """Run the GEMM against unit weights at offsets 0, N, 2N, ... until every
    column of A has been read out; compare C with deq(A) exactly."""
    M, K = A_bits.shape
    ref = bits_to_f64(expected_deq_bits(A_bits))
    A = inputs.from_bits(A_bits).to(DEV)
    off = 0
    while off < K or off == 0:
        packed = B.mx_pack_weight(unit_weight(N, K, off).to(DEV))
        C = B.mx_gemm(A, packed, N, plan=plan)
        torch.cuda.synchronize()
        got = bits_to_f64(inputs.bits(C.cpu()))
        cols = (np.arange(N) + off) % K
        want = ref[:, cols]
        bad = got != want          # -0 == +0
        if bad.any():
            i = np.argwhere(bad)[:5]
            raise AssertionError("%s off %d: %d of %d outputs differ from deq(A), e.g. %s" % (
                what, off, int(bad.sum()), bad.size,
                [(tuple(x), got[tuple(x)], want[tuple(x)]) for x in i]))
        off += N


ALL = list(inputs.WORKLOADS) + list(inputs.EXTRA_WORKLOADS)


@pytest.mark.parametrize("w", ALL, ids=[w.name for w in ALL])
@pytest.mark.parametrize("kind", ["workload", "adversarial"])
def test_workload_plan_quantises_a_bit_exactly(w, kind):
    """The plan the library picks for each measured workload, at its exact
    shape, on its seeded A and on adversarial rows of the same shape."""
    plan = B.mx_gemm_plan(w.M, w.N, w.K)
    say("quant-in-gemm", w.name, kind, plan)
    if kind == "workload":
        idx = [x.name for x in inputs.WORKLOADS].index(w.name) if w in inputs.WORKLOADS else None
        if idx is not None:
            A, _ = inputs.workload_inputs(idx, 1000)
        else:
            A, _ = inputs.shape_inputs(w.M, 8, w.K, seed=11)
        A_bits = inputs.bits(A)
    else:
        A_bits = adversarial(w.M, w.K, seed=w.M + w.K)
    check_extraction(A_bits, w.N, plan, "%s %s" % (w.name, kind))


# Explicit plans covering every activation mode and its variants: register
# quantisation with 1, 2 and 4 loaded row chunks, LDS-DMA tiles and the
# padded slab, the workgroup LDS quantiser, the pre-quantisation kernel,
# K splits with either finish, 16-wave workgroups, the K-looped stream mode,
# the quantiser-wave shared mode, the LDS-tiled tile mode.
PLANS = [
    dict(mb=1, nb=1, wn=1, wk=1, splits=1, amode=2),
    dict(mb=1, nb=1, wn=1, wk=4, splits=1, amode=2),
    dict(mb=1, nb=2, wn=1, wk=4, splits=7, amode=2),
    dict(mb=1, nb=2, wn=1, wk=4, splits=7, amode=2, finish=1),
    dict(mb=2, nb=1, wn=1, wk=8, splits=1, amode=2),
    dict(mb=1, nb=1, wn=2, wk=4, splits=3, amode=2),
    dict(mb=1, nb=2, wn=1, wk=16, splits=1, amode=2),
    dict(mb=1, nb=1, wn=1, wk=8, splits=1, amode=1),
    dict(mb=2, nb=2, wn=1, wk=1, splits=6, amode=1, finish=1),
    dict(mb=1, nb=1, wn=1, wk=1, splits=1, amode=0),
    dict(mb=2, nb=2, wn=2, wk=4, splits=1, amode=0),
    dict(mb=1, nb=1, wn=2, wk=4, splits=7, amode=0, finish=1),
    dict(mb=1, nb=1, wn=1, wk=1, splits=1, amode=4),
    dict(mb=1, nb=4, wn=1, wk=4, splits=1, amode=4),
    dict(mb=1, nb=2, wn=1, wk=16, splits=3, amode=4),
    dict(mb=1, nb=2, wn=1, wk=8, splits=2, amode=4, finish=1),
    dict(mb=1, nb=1, wn=4, wk=4, splits=1, amode=5),
    dict(mb=1, nb=2, wn=2, wk=2, splits=3, amode=5),
    dict(mb=8, nb=8, wn=4, wk=2, splits=1, amode=6),
    dict(mb=8, nb=4, wn=2, wk=2, splits=1, amode=6),
    dict(mb=4, nb=4, wn=4, wk=2, splits=1, amode=6),
    dict(mb=2, nb=2, wn=2, wk=2, splits=1, amode=6),
    dict(mb=2, nb=2, wn=2, wk=2, splits=2, amode=6),
]

SHAPES = [(5, 352), (13, 1088), (40, 2048), (70, 1536)]   # (M, K); N = K


def plan_id(p):
    return "mb%d_nb%d_wn%d_wk%d_s%d_a%d_f%d" % (p["mb"], p["nb"], p["wn"], p["wk"], p["splits"], p["amode"],
                                                p.get("finish", 0))


def accepted(M, N, K, plan):
    try:
        B.mx_gemm_workspace_bytes(M, N, K, plan)
        return True
    except B.MxError as e:
        assert e.code == B.MX_EPLAN
        return False


@pytest.mark.parametrize("plan", PLANS, ids=plan_id)
def test_explicit_plans_quantise_a_bit_exactly(plan):
    ran = 0
    for M, K in SHAPES:
        if not accepted(M, K, K, plan):
            continue
        say("quant-in-gemm plan", plan_id(plan), (M, K, K))
        A, _ = inputs.shape_inputs(M, 8, K, seed=M + K)
        check_extraction(inputs.bits(A), K, plan, "%s randn %s" % (plan_id(plan), (M, K)))
        check_extraction(adversarial(M, K, seed=3 * M + K), K, plan, "%s adversarial %s" % (plan_id(plan), (M, K)))
        ran += 1
    assert ran >= 1, "no shape accepted plan %s" % plan_id(plan)
