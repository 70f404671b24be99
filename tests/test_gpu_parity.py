"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

Every call goes through the C ABI (libmx4.so via the ctypes binding).  Codes
and e8m0 bytes must match the oracle bit for bit; C must satisfy, element by
element, |C_gpu - C_ref| <= 2 ulp_bf16(|C_ref|) + 1e-3 * rms(C_ref).
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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (the subnormal quantum at 0)."""
    a = np.abs(x).astype(np.float64)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return np.where(a > 0, np.ldexp(1.0, (e - 7).astype(np.int64)), np.ldexp(1.0, -133))


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_c_close(C_gpu_bits: np.ndarray, C_ref_bits: np.ndarray, what: str):
    g = bf16_bits_to_f64(C_gpu_bits)
    r = bf16_bits_to_f64(C_ref_bits)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    tol = 2.0 * ulp_bf16(r) + 1e-3 * rms
    err = np.abs(g - r)
    bad = err > tol
    assert np.isfinite(g).all(), what + ": non-finite output"
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d of %d outside tolerance, e.g. %s" % (
            what, int(bad.sum()), bad.size,
            [(tuple(i), g[tuple(i)], r[tuple(i)], tol[tuple(i)]) for i in idx]))


def to_dev(t: torch.Tensor) -> torch.Tensor:
    return t.to(DEV)


def gpu_bits(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return inputs.bits(t.cpu())


SENTINEL = -7.0


def guarded_c(M, N, ldc_pad=0):
    """C as the top-left M x N of a buffer filled with a sentinel: rows up to
    M rounded up to 64 plus 32 (past every row an M tile of the kernels can
    cover) and ldc_pad columns past N, so that a store outside C lands in
    this buffer and shows, instead of corrupting other memory."""
    rows = (M + 63) // 64 * 64 + 32
    Cbuf = torch.full((rows, N + ldc_pad), SENTINEL, dtype=torch.bfloat16, device=DEV)
    return Cbuf, Cbuf[:M, :N]


def assert_guard_intact(Cbuf, M, N):
    sent = inputs.bits(torch.tensor([SENTINEL], dtype=torch.bfloat16))[0]
    assert np.all(gpu_bits(Cbuf[M:]) == sent), "wrote past row M"
    if Cbuf.shape[1] > N:
        assert np.all(gpu_bits(Cbuf[:M, N:]) == sent), "wrote past column N"


def run_gemm(A_cpu, B_cpu, plan=None, ldc_pad=0, lda_pad=0):
    M, K = A_cpu.shape
    N = B_cpu.shape[0]
    if lda_pad:
        Abuf = torch.zeros((M, K + lda_pad), dtype=torch.bfloat16)
        Abuf[:, :K] = A_cpu
        A = to_dev(Abuf)[:, :K]
    else:
        A = to_dev(A_cpu)
    packed = B.mx_pack_weight(to_dev(B_cpu))
    Cbuf, C = guarded_c(M, N, ldc_pad)
    B.mx_gemm(A, packed, N, C=C, plan=plan)
    out = gpu_bits(C)
    assert_guard_intact(Cbuf, M, N)
    return out


# --------------------------------------------------------------------------
# activation quantiser (natural layout) and weight packer, bit-exact

@pytest.mark.parametrize("idx", range(len(inputs.WORKLOADS)), ids=[w.name for w in inputs.WORKLOADS])
@pytest.mark.parametrize("seed", [1000, 2000])
def test_quant_act_workloads_bit_exact(idx, seed):
    say("quant_act", inputs.WORKLOADS[idx].name, seed)
    A, _ = inputs.workload_inputs(idx, seed)
    codes, scales = B.mx_quant_act(to_dev(A))
    torch.cuda.synchronize()
    rc, rs = oracle.quant(inputs.bits(A))
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)


def adversarial_rows():
    """Rows of hand-worked groups, wide binade spreads, tiny and huge values."""
    import json, os, struct
    with open(os.path.join(os.path.dirname(__file__), "golden", "hand_groups.json")) as f:
        gs = json.load(f)["groups"]
    row = np.zeros(32 * len(gs), np.uint16)
    for gi, g in enumerate(gs):
        for k, v in g["values"].items():
            row[32 * gi + int(k)] = struct.unpack("<I", struct.pack("<f", v))[0] >> 16
    K = 32 * ((len(gs) + 7) // 8) * 8
    rows = np.zeros((3, K), np.uint16)
    rows[0, :row.size] = row
    rows[1, :row.size] = row[::-1]
    rows[2, :row.size] = row ^ 0x8000
    spread = inputs.bits(inputs.binade_spread(37, K, seed=5, lo=-140, hi=120))
    return np.concatenate([rows, spread])


def test_quant_act_adversarial_bit_exact():
    x = adversarial_rows()
    codes, scales = B.mx_quant_act(to_dev(inputs.from_bits(x)))
    torch.cuda.synchronize()
    rc, rs = oracle.quant(x)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)


def test_quant_act_strided_input():
    A, _ = inputs.shape_inputs(7, 8, 96, seed=3)
    buf = torch.zeros((7, 136), dtype=torch.bfloat16)
    buf[:, :96] = A
    codes, scales = B.mx_quant_act(to_dev(buf)[:, :96])
    torch.cuda.synchronize()
    rc, rs = oracle.quant(inputs.bits(A))
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)


@pytest.mark.parametrize("idx", range(len(inputs.WORKLOADS)), ids=[w.name for w in inputs.WORKLOADS])
def test_pack_unpack_workloads_bit_exact(idx):
    w = inputs.WORKLOADS[idx]
    say("pack", w.name)
    _, Bm = inputs.workload_inputs(idx, 1000)
    packed = B.mx_pack_weight(to_dev(Bm))
    codes, scales = B.mx_unpack_weight(packed, w.N, w.K)
    torch.cuda.synchronize()
    rc, rs = oracle.quant(inputs.bits(Bm))
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)


@pytest.mark.parametrize("N,K", [(1, 32), (33, 96), (70, 160), (129, 1088)])
def test_pack_unpack_ragged_bit_exact(N, K):
    Bm = inputs.binade_spread(N, K, seed=N + K, lo=-30, hi=30)
    packed = B.mx_pack_weight(to_dev(Bm))
    codes, scales = B.mx_unpack_weight(packed, N, K)
    torch.cuda.synchronize()
    rc, rs = oracle.quant(inputs.bits(Bm))
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)


@pytest.mark.parametrize("N,K", [(4, 64), (33, 96), (70, 160), (129, 1088), (2112, 7168)])
def test_import_weight_matches_pack(N, K):
    """Codes and scales quantised by the oracle, imported into the packed
    layout, give the very bytes mx_pack_weight writes (padding included),
    and unpack back to themselves."""
    Bm = inputs.binade_spread(N, K, seed=3 * N + K, lo=-20, hi=20)
    rc, rs = oracle.quant(inputs.bits(Bm))
    imported = B.mx_import_weight(to_dev(torch.from_numpy(rc)), to_dev(torch.from_numpy(rs)), N, K)
    packed = B.mx_pack_weight(to_dev(Bm))
    codes, scales = B.mx_unpack_weight(imported, N, K)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(imported.cpu().numpy(), packed.cpu().numpy())
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)


def test_import_weight_gemm():
    """A GEMM on an imported weight against the oracle on the same codes."""
    M, N, K = 16, 300, 1536
    A, Bm = inputs.shape_inputs(M, N, K, seed=99)
    rc, rs = oracle.quant(inputs.bits(Bm))
    packed = B.mx_import_weight(to_dev(torch.from_numpy(rc)), to_dev(torch.from_numpy(rs)), N, K)
    C = gpu_bits(B.mx_gemm(to_dev(A), packed, N))
    assert_c_close(C, oracle.gemm(inputs.bits(A), inputs.bits(Bm)), "imported weight")


def test_pack_adversarial_bit_exact():
    x = adversarial_rows()
    packed = B.mx_pack_weight(to_dev(inputs.from_bits(x)))
    codes, scales = B.mx_unpack_weight(packed, x.shape[0], x.shape[1])
    torch.cuda.synchronize()
    rc, rs = oracle.quant(x)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)


# --------------------------------------------------------------------------
# GEMM

@pytest.mark.parametrize("idx", range(len(inputs.WORKLOADS)), ids=[w.name for w in inputs.WORKLOADS])
@pytest.mark.parametrize("seed", [1000, 2000, 3000])
def test_gemm_workloads_full(idx, seed):
    """Every output of each measured workload under its production plan."""
    w = inputs.WORKLOADS[idx]
    say("gemm", w.name, seed, B.mx_gemm_plan(w.M, w.N, w.K))
    A, Bm = inputs.workload_inputs(idx, seed)
    C = run_gemm(A, Bm)
    ref = oracle.gemm(inputs.bits(A), inputs.bits(Bm))
    assert_c_close(C, ref, w.name)


@pytest.mark.parametrize("w", inputs.EXTRA_WORKLOADS, ids=[w.name for w in inputs.EXTRA_WORKLOADS])
@pytest.mark.parametrize("seed", [1, 2])
def test_gemm_extra_workloads_full(w, seed):
    say("gemm", w.name, seed, B.mx_gemm_plan(w.M, w.N, w.K))
    A, Bm = inputs.shape_inputs(w.M, w.N, w.K, seed=seed)
    C = run_gemm(A, Bm)
    assert_c_close(C, oracle.gemm(inputs.bits(A), inputs.bits(Bm)), w.name)


SMALL_SHAPES = [
    (1, 32, 32), (4, 96, 128), (5, 200, 320), (17, 130, 96), (33, 64, 64),
    (32, 96, 512), (40, 100, 2048), (70, 300, 1536), (16, 64, 7168), (65, 37, 256),
]

PLANS = [
    dict(mb=1, nb=1, wn=1, wk=1, splits=1, amode=0),
    dict(mb=1, nb=2, wn=1, wk=4, splits=1, amode=0),
    dict(mb=1, nb=1, wn=1, wk=8, splits=2, amode=0),
    dict(mb=2, nb=1, wn=2, wk=2, splits=1, amode=0),
    dict(mb=1, nb=2, wn=2, wk=4, splits=3, amode=0),
    dict(mb=2, nb=2, wn=2, wk=4, splits=1, amode=0),
    dict(mb=1, nb=1, wn=1, wk=16, splits=1, amode=0),
    dict(mb=1, nb=1, wn=1, wk=1, splits=1, amode=1),
    dict(mb=2, nb=2, wn=1, wk=1, splits=6, amode=1),
    dict(mb=1, nb=1, wn=2, wk=8, splits=4, amode=1),
    dict(mb=2, nb=1, wn=2, wk=2, splits=2, amode=1),
    dict(mb=2, nb=2, wn=1, wk=16, splits=1, amode=1),
    dict(mb=1, nb=1, wn=1, wk=1, splits=1, amode=2),
    dict(mb=1, nb=1, wn=1, wk=4, splits=1, amode=2),
    dict(mb=2, nb=2, wn=2, wk=2, splits=3, amode=2),
    dict(mb=1, nb=2, wn=1, wk=16, splits=1, amode=2),
    dict(mb=2, nb=1, wn=1, wk=8, splits=2, amode=2),
    dict(mb=1, nb=1, wn=2, wk=4, splits=7, amode=2),
    dict(mb=1, nb=1, wn=2, wk=4, splits=7, amode=0, finish=1),
    dict(mb=2, nb=2, wn=1, wk=1, splits=6, amode=1, finish=1),
    dict(mb=1, nb=2, wn=2, wk=4, splits=3, amode=2, finish=1),
    dict(mb=2, nb=1, wn=1, wk=16, splits=2, amode=0, finish=1),
    dict(mb=1, nb=1, wn=1, wk=1, splits=1, amode=4),
    dict(mb=1, nb=2, wn=1, wk=4, splits=1, amode=4),
    dict(mb=1, nb=4, wn=1, wk=8, splits=1, amode=4),
    dict(mb=1, nb=2, wn=1, wk=16, splits=3, amode=4),
    dict(mb=1, nb=4, wn=1, wk=2, splits=2, amode=4, finish=1),
    dict(mb=1, nb=1, wn=2, wk=2, splits=1, amode=5),
    dict(mb=1, nb=1, wn=4, wk=4, splits=1, amode=5),
    dict(mb=1, nb=2, wn=2, wk=2, splits=3, amode=5),
    dict(mb=1, nb=2, wn=4, wk=4, splits=2, amode=5),
    dict(mb=8, nb=8, wn=4, wk=2, splits=1, amode=6),
    dict(mb=4, nb=8, wn=2, wk=2, splits=1, amode=6),
    dict(mb=8, nb=4, wn=2, wk=2, splits=1, amode=6),
    dict(mb=4, nb=4, wn=2, wk=2, splits=1, amode=6),
    dict(mb=4, nb=4, wn=4, wk=2, splits=1, amode=6),
    dict(mb=2, nb=2, wn=2, wk=2, splits=1, amode=6),
    dict(mb=2, nb=2, wn=2, wk=2, splits=3, amode=6),
    dict(mb=8, nb=4, wn=2, wk=2, splits=2, amode=6),
]

# (8192 x 8192 x 512: a 32 x 32 grid of 256 x 256 tiles, four rounds per XCD, placed per round)
# M from 128 takes the 128 x 128 and 64 x 64 tiles (130 and 200: ragged M); 777 x 4100, 1024 x 2880 and
# 512 x 2112 place runs of consecutive tiles on the XCDs (their tile counts split into no good rectangles)
LARGE_M_SHAPES = [(1024, 4096, 4096), (2048, 7168, 2048), (384, 7168, 7168), (777, 4100, 4160), (8192, 8192, 512),
                  (256, 4096, 4096), (130, 7168, 7168), (200, 7168, 2048), (1024, 2880, 2048), (512, 2112, 7168),
                  (96, 3072, 4096), (128, 2112, 5120), (160, 2880, 3072)]


@pytest.mark.parametrize("shape", LARGE_M_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_large_m_takes_the_tile_mode(shape):
    """Shapes from M = 96 up run the K-looped tile mode by the library's own plan;
    sampled rows (the first, the last and 14 random ones) by sampled columns
    (the first 4, the last 4 and 60 random ones) of C against the oracle's
    product of exactly those rows of A and columns of B."""
    M, N, K = shape
    plan = B.mx_gemm_plan(M, N, K)
    assert plan["amode"] == B.MX_AMODE_TILE, plan
    say("large M", shape, plan_id(plan))
    gen = torch.Generator("cpu").manual_seed(M + N + K)
    A = inputs.bf16_randn(M, K, gen)
    Bm = inputs.bf16_randn(N, K, gen)
    C = gpu_bits(B.mx_gemm(to_dev(A), B.mx_pack_weight(to_dev(Bm)), N))
    rng = np.random.default_rng(M + N)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 14)]))
    cols = np.unique(np.concatenate([np.arange(4), np.arange(N - 4, N), rng.integers(0, N, 60)]))
    ref = oracle.gemm(np.ascontiguousarray(inputs.bits(A)[rows]), np.ascontiguousarray(inputs.bits(Bm)[cols]))
    assert_c_close(C[np.ix_(rows, cols)], ref, "%s %s" % (shape, plan_id(plan)))


# Between the grid's M values the shared mode runs where its grid fits one
# round on the 256 CUs: three MFMA waves (160 x 3072), four (288 x 3072,
# 200 x 4096: ragged M), four with a ragged last N tile (320 x 2880)
ROUND_SHAPES = [((160, 3072, 1536), 3), ((288, 3072, 1536), 4), ((200, 4096, 1024), 4), ((320, 2880, 1536), 4)]


@pytest.mark.parametrize("case", ROUND_SHAPES, ids=lambda c: "x".join(map(str, c[0])))
def test_mid_m_shared_mode_in_one_round(case):
    """Off-grid M from 5 M blocks takes the shared mode with the MFMA waves
    whose grid fits one round; sampled rows by sampled columns of C against
    the oracle's product of exactly those rows and columns."""
    (M, N, K), wn = case
    plan = B.mx_gemm_plan(M, N, K)
    assert plan["amode"] == B.MX_AMODE_SHARED and plan["wn"] == wn, plan
    assert -(-M // 32) * -(-(-(-N // 32)) // wn) <= 256
    say("one round", (M, N, K), plan_id(plan))
    gen = torch.Generator("cpu").manual_seed(M + N + K)
    A = inputs.bf16_randn(M, K, gen)
    Bm = inputs.bf16_randn(N, K, gen)
    C = gpu_bits(B.mx_gemm(to_dev(A), B.mx_pack_weight(to_dev(Bm)), N))
    rng = np.random.default_rng(M + N)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 14)]))
    cols = np.unique(np.concatenate([np.arange(4), np.arange(N - 4, N), rng.integers(0, N, 60)]))
    ref = oracle.gemm(np.ascontiguousarray(inputs.bits(A)[rows]), np.ascontiguousarray(inputs.bits(Bm)[cols]))
    assert_c_close(C[np.ix_(rows, cols)], ref, "%s %s" % ((M, N, K), plan_id(plan)))


# The a16wfp4 product (amode 3) against its own oracle.
PLANS_A16W4 = [
    dict(mb=1, nb=1, wn=1, wk=1, splits=1, amode=3),
    dict(mb=1, nb=1, wn=1, wk=4, splits=1, amode=3),
    dict(mb=1, nb=2, wn=2, wk=2, splits=3, amode=3),
    dict(mb=2, nb=1, wn=1, wk=8, splits=2, amode=3),
    dict(mb=1, nb=1, wn=2, wk=8, splits=7, amode=3, finish=1),
]


def plan_id(p):
    return "mb%d_nb%d_wn%d_wk%d_s%d_a%d_f%d" % (p["mb"], p["nb"], p["wn"], p["wk"], p["splits"], p["amode"],
                                                p.get("finish", 0))


def plan_runs(M, N, K, plan):
    try:
        B.mx_gemm_workspace_bytes(M, N, K, plan)
        return True
    except B.MxError as e:
        assert e.code == B.MX_EPLAN
        return False


@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemm_small_shapes_auto_plan(shape):
    M, N, K = shape
    say("gemm small", shape, B.mx_gemm_plan(M, N, K))
    A, Bm = inputs.shape_inputs(M, N, K, seed=M * 7 + N + K)
    C = run_gemm(A, Bm)
    assert_c_close(C, oracle.gemm(inputs.bits(A), inputs.bits(Bm)), str(shape))


@pytest.mark.parametrize("plan", PLANS, ids=plan_id)
@pytest.mark.parametrize("shape", [(5, 200, 320), (70, 300, 1536), (33, 130, 2048), (9, 70, 352)],
                         ids=lambda s: "x".join(map(str, s)))
def test_gemm_explicit_plans(shape, plan):
    M, N, K = shape
    if not plan_runs(M, N, K, plan):
        pytest.skip("plan outside the register / LDS budget for this shape")
    say("gemm plan", shape, plan_id(plan))
    A, Bm = inputs.shape_inputs(M, N, K, seed=11 + M + N)
    C = run_gemm(A, Bm, plan=plan)
    assert_c_close(C, oracle.gemm(inputs.bits(A), inputs.bits(Bm)), "%s %s" % (shape, plan_id(plan)))


@pytest.mark.parametrize("plan", PLANS + PLANS_A16W4, ids=plan_id)
@pytest.mark.parametrize("shape", [(5, 200, 320), (33, 130, 2048), (9, 70, 352), (40, 100, 2048)],
                         ids=lambda s: "x".join(map(str, s)))
def test_gemm_writes_nothing_outside_c(shape, plan):
    """Every plan leaves the memory around C alone: the rows past M of its
    last M tile and the columns past N of its last N tile are masked (C sits
    in a sentinel-filled buffer 128 columns wider, ldc = N + 128)."""
    M, N, K = shape
    if not plan_runs(M, N, K, plan):
        pytest.skip("plan outside the register / LDS budget for this shape")
    say("gemm guard", shape, plan_id(plan))
    A, Bm = inputs.shape_inputs(M, N, K, seed=3 + M + N)
    Ad = to_dev(A)
    packed = B.mx_pack_weight(to_dev(Bm))
    Cbuf, C = guarded_c(M, N, 128)
    B.mx_gemm(Ad, packed, N, C=C, plan=plan)
    assert_guard_intact(Cbuf, M, N)
    ref = oracle.gemm_a16w4 if plan["amode"] == 3 else oracle.gemm
    assert_c_close(gpu_bits(C), ref(inputs.bits(A), inputs.bits(Bm)), "%s %s" % (shape, plan_id(plan)))


# one plan of every activation mode (None: the library's own) for strided A
# and C: lda = K + 24 elements, ldc = N + 5
STRIDE_PLANS = [None,
                dict(mb=1, nb=2, wn=1, wk=4, splits=1, amode=0),
                dict(mb=2, nb=1, wn=2, wk=2, splits=2, amode=1),
                dict(mb=1, nb=1, wn=1, wk=4, splits=1, amode=2),
                dict(mb=1, nb=2, wn=1, wk=4, splits=1, amode=4),
                dict(mb=1, nb=1, wn=3, wk=4, splits=1, amode=5),
                dict(mb=8, nb=4, wn=2, wk=2, splits=1, amode=6),
                dict(mb=4, nb=8, wn=2, wk=2, splits=1, amode=6),
                dict(mb=2, nb=2, wn=2, wk=2, splits=1, amode=6),
                dict(mb=4, nb=4, wn=4, wk=2, splits=2, amode=6)]


@pytest.mark.parametrize("plan", STRIDE_PLANS, ids=lambda p: "auto" if p is None else plan_id(p))
def test_gemm_binade_spread_and_strides(plan):
    M, N, K = 19, 75, 640
    if plan is not None and not plan_runs(M, N, K, plan):
        pytest.skip("plan outside the register / LDS budget for this shape")
    A = inputs.binade_spread(M, K, seed=21, lo=-10, hi=10)
    Bm = inputs.binade_spread(N, K, seed=22, lo=-10, hi=10)
    say("gemm strides", "auto" if plan is None else plan_id(plan))
    C = run_gemm(A, Bm, plan=plan, lda_pad=24, ldc_pad=5)
    assert_c_close(C, oracle.gemm(inputs.bits(A), inputs.bits(Bm)), "binades %s" % plan)


def test_gemm_closed_form_all_ones():
    M, N, K = 3, 40, 7168
    A = torch.ones((M, K), dtype=torch.bfloat16)
    Bm = torch.ones((N, K), dtype=torch.bfloat16)
    C = run_gemm(A, Bm)
    assert np.all(C == inputs.bits(torch.tensor([float(K)], dtype=torch.bfloat16))[0])


def test_gemm_zero_inputs():
    M, N, K = 8, 64, 256
    C = run_gemm(torch.zeros((M, K), dtype=torch.bfloat16), torch.zeros((N, K), dtype=torch.bfloat16))
    assert np.all(C == 0)


def test_split_k_deterministic_and_consistent():
    M, N, K = 16, 2112, 7168
    A, Bm = inputs.shape_inputs(M, N, K, seed=77)
    Ad = to_dev(A)
    packed = B.mx_pack_weight(to_dev(Bm))
    plan = B.mx_gemm_plan(M, N, K)
    assert plan["splits"] > 1
    ws = B.new_workspace(M, N, K, plan, device=DEV)
    c1 = gpu_bits(B.mx_gemm(Ad, packed, N, plan=plan, workspace=ws))
    c2 = gpu_bits(B.mx_gemm(Ad, packed, N, plan=plan, workspace=ws))
    np.testing.assert_array_equal(c1, c2)
    # another activation mode and split count: register quantisation, 4 splits
    other = dict(mb=1, nb=2, wn=1, wk=4, splits=4, amode=2, finish=0)
    assert other != plan
    c3 = gpu_bits(B.mx_gemm(Ad, packed, N, plan=other))
    ref = oracle.gemm(inputs.bits(A), inputs.bits(Bm))
    assert_c_close(c1, ref, "split %d" % plan["splits"])
    assert_c_close(c3, ref, "split 4")
    # the tile mode's K splits (4 steps a split start): deterministic, and the
    # same C as its one-split plan up to the fp32 order of the partial sums
    tile = dict(mb=2, nb=2, wn=2, wk=2, splits=5, amode=6, finish=0)
    c4 = gpu_bits(B.mx_gemm(Ad, packed, N, plan=tile))
    c5 = gpu_bits(B.mx_gemm(Ad, packed, N, plan=tile))
    np.testing.assert_array_equal(c4, c5)
    assert_c_close(c4, ref, "tile split 5")


def test_gemm_streams_and_reuse_of_workspace():
    """Two shapes in a row on a side stream, sharing one workspace buffer."""
    s = torch.cuda.Stream()
    shapes = [(16, 2112, 7168), (70, 300, 1536)]
    ws_bytes = max(B.mx_gemm_workspace_bytes(*sh) for sh in shapes)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    outs = []
    with torch.cuda.stream(s):
        for (M, N, K) in shapes:
            A, Bm = inputs.shape_inputs(M, N, K, seed=M + N)
            Ad, Bd = to_dev(A), to_dev(Bm)
            packed = B.mx_pack_weight(Bd, stream=s)
            C = B.mx_gemm(Ad, packed, N, workspace=ws, stream=s)
            outs.append((C, A, Bm))
    s.synchronize()
    for C, A, Bm in outs:
        assert_c_close(inputs.bits(C.cpu()), oracle.gemm(inputs.bits(A), inputs.bits(Bm)), "stream")


LAST_ARRIVAL_CASES = [
    ((16, 2112, 7168), dict(mb=1, nb=1, wn=2, wk=4, splits=7, amode=0)),
    ((16, 2112, 7168), dict(mb=1, nb=2, wn=1, wk=8, splits=14, amode=2)),
    ((33, 130, 2048), dict(mb=2, nb=1, wn=1, wk=2, splits=8, amode=1)),
    ((70, 300, 1536), dict(mb=1, nb=1, wn=1, wk=4, splits=3, amode=0)),
    ((9, 70, 352), dict(mb=1, nb=1, wn=1, wk=1, splits=6, amode=2)),
]


@pytest.mark.parametrize("case", LAST_ARRIVAL_CASES, ids=lambda c: "x".join(map(str, c[0])) + "_s%d" % c[1]["splits"])
def test_split_k_last_arrival_matches_reduce_kernel(case):
    """The in-GEMM finish sums the same partials in the same order as the
    reduction kernel: bit-identical C, within tolerance of the oracle, and
    the arrival counters are back at zero after every call."""
    (M, N, K), plan = case
    if not plan_runs(M, N, K, dict(plan, finish=1)):
        pytest.skip("plan outside the register / LDS budget for this shape")
    say("last arrival", (M, N, K), plan)
    A, Bm = inputs.shape_inputs(M, N, K, seed=5 + M + K)
    Ad = to_dev(A)
    packed = B.mx_pack_weight(to_dev(Bm))
    ref_kernel = gpu_bits(B.mx_gemm(Ad, packed, N, plan=dict(plan, finish=0)))
    ws = B.new_workspace(M, N, K, dict(plan, finish=1), device=DEV)
    outs = [B.mx_gemm(Ad, packed, N, plan=dict(plan, finish=1), workspace=ws) for _ in range(5)]
    torch.cuda.synchronize()
    assert int(ws[:16384].count_nonzero()) == 0, "arrival counters not returned to zero"
    for C in outs:
        np.testing.assert_array_equal(gpu_bits(C), ref_kernel)
    assert_c_close(ref_kernel, oracle.gemm(inputs.bits(A), inputs.bits(Bm)), "last arrival")


def test_split_k_last_arrival_workspace_across_shapes():
    """One zero-filled workspace serves a sequence of shapes and plans, with
    partials of one shape landing where another's activation codes were."""
    seq = [((16, 2112, 7168), dict(mb=1, nb=1, wn=2, wk=4, splits=7, amode=0, finish=1)),
           ((70, 300, 1536), dict(mb=2, nb=1, wn=1, wk=4, splits=3, amode=1, finish=1)),
           ((16, 2112, 7168), dict(mb=1, nb=1, wn=2, wk=4, splits=7, amode=0, finish=1)),
           ((33, 130, 2048), dict(mb=1, nb=1, wn=1, wk=8, splits=4, amode=2, finish=1)),
           ((70, 300, 1536), dict(mb=2, nb=1, wn=1, wk=4, splits=3, amode=1, finish=1))]
    ws = torch.zeros(max(B.mx_gemm_workspace_bytes(*sh, p) for sh, p in seq), dtype=torch.uint8, device=DEV)
    data = {}
    for (M, N, K), plan in seq:
        if (M, N, K) not in data:
            A, Bm = inputs.shape_inputs(M, N, K, seed=M * N)
            data[(M, N, K)] = (A, Bm, to_dev(A), B.mx_pack_weight(to_dev(Bm)))
        A, Bm, Ad, packed = data[(M, N, K)]
        say("workspace sequence", (M, N, K), plan)
        C = gpu_bits(B.mx_gemm(Ad, packed, N, plan=plan, workspace=ws))
        assert_c_close(C, oracle.gemm(inputs.bits(A), inputs.bits(Bm)), str((M, N, K)))
    assert int(ws[:16384].count_nonzero()) == 0


def test_gemm_graph_capture_replays_match_eager():
    """mx_gemm enqueues kernels only (no allocation, synchronisation or
    memset), so a caller can capture calls into a HIP graph.  Three shapes
    (one launch, pre-quantised A, split-K) are captured once; the graph is
    replayed several times with eager work and synchronisation in between,
    with new activations copied in before some replays, and every replay is
    compared bit-for-bit with eager calls on the same inputs."""
    cases = []
    for (M, N, K) in [(32, 4096, 512), (64, 640, 2048), (16, 2112, 7168)]:
        A, Bm = inputs.shape_inputs(M, N, K, seed=M + 3 * N)
        Ad = to_dev(A)
        packed = B.mx_pack_weight(to_dev(Bm))
        C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        ws = B.new_workspace(M, N, K, device=DEV)
        cases.append((M, N, K, Ad, packed, C, ws))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for (M, N, K, Ad, packed, C, ws) in cases:
            B.mx_gemm(Ad, packed, N, C=C, workspace=ws, stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    for replay in range(4):
        if replay == 2:   # new activations, same buffers
            for (M, N, K, Ad, packed, C, ws) in cases:
                Ad.copy_(to_dev(inputs.shape_inputs(M, N, K, seed=77 + M)[0]))
        for (_, _, _, _, _, C, _) in cases:
            C.fill_(7.0)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (M, N, K, Ad, packed, C, ws) in cases:
            eager = gpu_bits(B.mx_gemm(Ad, packed, N))
            np.testing.assert_array_equal(gpu_bits(C), eager, err_msg="replay %d shape %s" % (replay, (M, N, K)))



# ---------------------------------------------------------------------------
# a16wfp4: C = A (bf16, not quantised) x dequant(B)^T

def run_a16w4(A, Bm, plan=None):
    Ad = to_dev(A)
    packed = B.mx_pack_weight(to_dev(Bm))
    if plan is None:
        C = B.mx_gemm_a16w4(Ad, packed, Bm.shape[0])
    else:
        C = B.mx_gemm(Ad, packed, Bm.shape[0], plan=plan)
    return gpu_bits(C)


@pytest.mark.parametrize("idx", range(len(inputs.WORKLOADS)), ids=[w.name for w in inputs.WORKLOADS])
def test_a16w4_workloads_full(idx):
    w = inputs.WORKLOADS[idx]
    say("a16w4", w.name, B.mx_gemm_a16w4_plan(w.M, w.N, w.K))
    A, Bm = inputs.workload_inputs(idx, 2000)
    C = run_a16w4(A, Bm)
    assert_c_close(C, oracle.gemm_a16w4(inputs.bits(A), inputs.bits(Bm)), "a16w4 " + w.name)


@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_a16w4_small_shapes(shape):
    M, N, K = shape
    A, Bm = inputs.shape_inputs(M, N, K, seed=M + 2 * N + K)
    C = run_a16w4(A, Bm)
    assert_c_close(C, oracle.gemm_a16w4(inputs.bits(A), inputs.bits(Bm)), "a16w4 " + str(shape))


@pytest.mark.parametrize("plan", PLANS_A16W4, ids=plan_id)
@pytest.mark.parametrize("shape", [(5, 200, 320), (70, 300, 1536), (9, 70, 352)], ids=lambda s: "x".join(map(str, s)))
def test_a16w4_explicit_plans(shape, plan):
    M, N, K = shape
    if not plan_runs(M, N, K, plan):
        pytest.skip("plan outside the register / LDS budget for this shape")
    say("a16w4 plan", shape, plan_id(plan))
    A, Bm = inputs.shape_inputs(M, N, K, seed=31 + M + N)
    C = run_a16w4(A, Bm, plan)
    assert_c_close(C, oracle.gemm_a16w4(inputs.bits(A), inputs.bits(Bm)), "a16w4 " + plan_id(plan))


@pytest.mark.parametrize("lo_a,hi_a,lo_b,hi_b", [(-20, 20, -20, 20), (-10, 10, -133, -120), (-110, -90, 80, 100)],
                         ids=["spread", "tiny_weight", "tiny_act_huge_weight"])
def test_a16w4_binades(lo_a, hi_a, lo_b, hi_b):
    """Weight groups down to scale byte 0 widen to bf16 subnormals (the
    convert must keep them); wide exponent ranges on both sides."""
    M, N, K = 12, 96, 512
    A = inputs.binade_spread(M, K, seed=41, lo=lo_a, hi=hi_a)
    Bm = inputs.binade_spread(N, K, seed=42, lo=lo_b, hi=hi_b)
    C = run_a16w4(A, Bm)
    ref = oracle.gemm_a16w4(inputs.bits(A), inputs.bits(Bm))
    assert np.any(ref != 0)
    assert_c_close(C, ref, "a16w4 binades")


def test_a16w4_representable_weight_is_exact_matmul():
    """Integer activations in [-16, 16] against an MXFP4-representable weight
    with scales 2^-1..2^1: every product and partial sum is a multiple of
    1/4 below 2^13, exact in fp32, so C is bit-identical to the oracle."""
    M, N, K = 32, 64, 64
    rng = np.random.default_rng(45)
    A = torch.from_numpy(rng.integers(-16, 17, (M, K)).astype(np.float32)).to(torch.bfloat16)
    Bm = inputs.from_bits(oracle_representable(N, K))
    C = run_a16w4(A, Bm)
    np.testing.assert_array_equal(C, oracle.gemm_a16w4(inputs.bits(A), inputs.bits(Bm)))


def oracle_representable(rows, K):
    """bf16 bits of an MXFP4-representable matrix (codes and bytes chosen at
    random, values decoded with the oracle)."""
    rng = np.random.default_rng(44)
    codes = rng.integers(0, 16, (rows, K)).astype(np.uint8)
    codes[:, ::32] = 7                      # every group reaches 6 * 2^s: the rule keeps s
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(126, 129, (rows, K // 32)).astype(np.uint8)
    vals = oracle.dequant(packed, scales)
    return inputs.bits(torch.from_numpy(vals).to(torch.bfloat16))


# ---------------------------------------------------------------------------
# Sizes at the 32-bit addressing limits (rows * K * 2 < 2^31 per operand),
# checked on sampled outputs the oracle computes one row / column at a time.

def gpu_randn_bf16(rows, cols, seed, scale=1.0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return (torch.randn(rows, cols, generator=g, device=DEV, dtype=torch.float32) * scale).to(torch.bfloat16)


@pytest.mark.parametrize("M,N,K,sample", [
    (64, 32768, 32736, "n"),     # a 1 GiB bf16 weight (rows * K just under 2^30), K % 64 == 32
    (32768, 512, 1024, "m"),     # a 64 MiB activation, many M tiles
    (32, 32, 1 << 22, "all"),    # K = 4M: 65536 K steps, 1024 splits
    (1, 16384, 65504, "n"),      # one row against a 2 GiB-limit weight
], ids=["bigN", "bigM", "bigK", "m1_bigNK"])
def test_gemm_limit_sizes_sampled(M, N, K, sample):
    say("limit size", (M, N, K), B.mx_gemm_plan(M, N, K))
    Ad = gpu_randn_bf16(M, K, seed=M + K)
    Bd = gpu_randn_bf16(N, K, seed=N + 7 * K)
    packed = B.mx_pack_weight(Bd)
    C = B.mx_gemm(Ad, packed, N)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M + N + K)
    if sample == "n":
        cols = np.sort(rng.choice(N, size=min(N, 48), replace=False))
        ref = oracle.gemm(inputs.bits(Ad.cpu()), inputs.bits(Bd[torch.from_numpy(cols).to(DEV)].cpu()))
        got = inputs.bits(C[:, torch.from_numpy(cols).to(DEV)].cpu())
    elif sample == "m":
        rows = np.sort(rng.choice(M, size=min(M, 48), replace=False))
        ref = oracle.gemm(inputs.bits(Ad[torch.from_numpy(rows).to(DEV)].cpu()), inputs.bits(Bd.cpu()))
        got = inputs.bits(C[torch.from_numpy(rows).to(DEV)].cpu())
    else:
        ref = oracle.gemm(inputs.bits(Ad.cpu()), inputs.bits(Bd.cpu()))
        got = inputs.bits(C.cpu())
    assert_c_close(got, ref, "limit size %s" % ((M, N, K),))
    del Ad, Bd, packed, C
    torch.cuda.empty_cache()


def test_gemm_from_several_host_threads():
    """Four host threads, each with its own stream, shapes and workspace,
    call mx_gemm repeatedly (each thread keeps its own cache of prepared
    calls); every result matches the oracle."""
    import threading
    shapes = [(32, 4096, 512), (16, 2112, 7168), (64, 640, 2048), (5, 200, 320)]
    data = []
    for (M, N, K) in shapes:
        A, Bm = inputs.shape_inputs(M, N, K, seed=900 + M + N)
        data.append((M, N, K, to_dev(A), B.mx_pack_weight(to_dev(Bm)),
                     oracle.gemm(inputs.bits(A), inputs.bits(Bm))))
    torch.cuda.synchronize()
    errors = []

    def worker(idx):
        try:
            M, N, K, Ad, packed, ref = data[idx]
            s = torch.cuda.Stream()
            ws = B.new_workspace(M, N, K, device=DEV)
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                outs = [B.mx_gemm(Ad, packed, N, workspace=ws, stream=s) for _ in range(20)]
            s.synchronize()
            for C in outs:
                assert_c_close(inputs.bits(C.cpu()), ref, "thread %d" % idx)
        except Exception as e:   # reported from the main thread
            errors.append((idx, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(shapes))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors


@pytest.mark.gpu
def test_random_shapes_and_plans():
    """150 seeded random cases: M in [1, ~315], N in [1, ~720], K a multiple
    of 32 up to 3072, half of them with one binade per 32-element group
    (2^-20 .. 2^20).  Each case checks the activation codes and scales
    bit-exactly, C of the chosen plan and of one random plan the planner
    accepts (any activation mode, split and finish) to the C tolerance, and
    the a16wfp4 product against its oracle."""
    import itertools
    import random
    rng = random.Random(20261203)
    fields = ["mb", "nb", "wn", "wk", "splits", "amode", "finish"]
    cands = list(itertools.product([1, 2], [1, 2], [1, 2], [1, 2, 4, 8, 16], [1, 2, 3, 4, 7, 8], [0, 1, 2], [0, 1]))
    for case in range(150):
        M = max(1, int(round(2 ** rng.uniform(0, 8.3))))
        N = max(1, int(round(2 ** rng.uniform(0, 9.5))))
        K = 32 * rng.randint(1, 96)
        g = torch.Generator().manual_seed(rng.randrange(1 << 30))
        A = torch.randn(M, K, generator=g)
        Bf = torch.randn(N, K, generator=g)
        if rng.random() < 0.5:
            A = A * torch.pow(2.0, torch.randint(-20, 21, (M, K // 32), generator=g).float()).repeat_interleave(32, 1)
            Bf = Bf * torch.pow(2.0, torch.randint(-20, 21, (N, K // 32), generator=g).float()).repeat_interleave(32, 1)
        A, Bm = A.to(torch.bfloat16), Bf.to(torch.bfloat16)
        Ab, Bb = inputs.bits(A), inputs.bits(Bm)
        plans = [None]
        for _ in range(50):
            pl = dict(zip(fields, rng.choice(cands)))
            if pl["splits"] == 1 and pl["finish"] == 1:
                continue
            try:
                B.mx_gemm_workspace_bytes(M, N, K, pl)
            except B.MxError:
                continue
            plans.append(pl)
            break
        say("random case %d: M=%d N=%d K=%d plans %s" % (case, M, N, K, plans))
        Ad, Bd = to_dev(A), to_dev(Bm)
        packed = B.mx_pack_weight(Bd)
        ref = oracle.gemm(Ab, Bb)
        for pl in plans:
            assert_c_close(gpu_bits(B.mx_gemm(Ad, packed, N, plan=pl)), ref,
                           "random case %d %s plan %s" % (case, (M, N, K), pl))
        codes, scales = B.mx_quant_act(Ad)
        rc, rs = oracle.quant(Ab)
        torch.cuda.synchronize()
        assert np.array_equal(codes.cpu().numpy(), rc) and np.array_equal(scales.cpu().numpy(), rs), \
            "random case %d: activation codes or scales differ" % case
        assert_c_close(gpu_bits(B.mx_gemm_a16w4(Ad, packed, N)), oracle.gemm_a16w4(Ab, Bb),
                       "random case %d %s a16wfp4" % (case, (M, N, K)))


@pytest.mark.gpu
@pytest.mark.parametrize("scale_exp", [0, -67], ids=["normal", "subnormal"])
def test_gemm_bf16_rounding_ties_bit_exact(scale_exp):
    """The epilogue's fp32 -> bf16 rounding, bit-exactly: with A and B made of
    0 and 2^e (e = 0, or -67 so that each product is 2^-134, below bf16's
    normal range), C[m, n] = 2^(2e) * (count of common ones) is an exact fp32
    sum, and the counts 200..512 hit bf16 ties (odd counts above 256, and odd
    multiples of 2^-134, halfway between bf16 subnormals).  Round to nearest
    even must give the oracle's once-rounded result exactly, on every plan
    mode and split."""
    M, N, K = 8, 160, 512
    v = 2.0 ** scale_exp
    rows_a = [200 + 39 * m for m in range(M)]                 # ones in A's first k_m columns
    rows_b = [201 + 2 * n for n in range(N)]                  # ones in B's first k_n columns
    A = torch.zeros(M, K)
    for m, k in enumerate(rows_a):
        A[m, :min(k, K)] = v
    Bf = torch.zeros(N, K)
    for n, k in enumerate(rows_b):
        Bf[n, :min(k, K)] = v
    A, Bm = A.to(torch.bfloat16), Bf.to(torch.bfloat16)
    ref = oracle.gemm(inputs.bits(A), inputs.bits(Bm))
    Ad, packed = to_dev(A), B.mx_pack_weight(to_dev(Bm))
    for plan in [None, dict(mb=1, nb=1, wn=1, wk=4, splits=1, amode=0, finish=0),
                 dict(mb=1, nb=1, wn=1, wk=2, splits=1, amode=1, finish=0),
                 dict(mb=1, nb=1, wn=1, wk=1, splits=4, amode=2, finish=0),
                 dict(mb=1, nb=1, wn=1, wk=2, splits=2, amode=2, finish=1)]:
        say("rounding ties, scale 2^%d, plan %s" % (scale_exp, plan))
        got = gpu_bits(B.mx_gemm(Ad, packed, N, plan=plan))
        assert np.array_equal(got, ref), "plan %s: %d outputs differ from round-to-nearest-even" % (
            plan, int((got != ref).sum()))
    got16 = gpu_bits(B.mx_gemm_a16w4(Ad, packed, N))
    assert np.array_equal(got16, oracle.gemm_a16w4(inputs.bits(A), inputs.bits(Bm)))
