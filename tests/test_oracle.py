"""Pins of the CPU oracle against things other than itself (CPU only).

* hand-worked groups (tests/golden/hand_groups.json, worked out by hand from
  the quantisation rule of the kernelindex.com amd-mxfp4-mm pages);
* an exact, separately formulated pure-Python brute force (oracle.bruteforce):
  encoder and scale byte over every finite bf16 value, whole GEMMs on tiny
  shapes with bit-identical C;
* closed forms (all-ones, hand sums, MXFP4-representable inputs whose product
  is a textbook fp64 matmul) and invariants of the encoding.
"""
import json
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import bruteforce as bf
from microscaled_mxfp4_block_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_groups.json")
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def f2bf(v: float) -> int:
    u = struct.unpack("<I", struct.pack("<f", v))[0]
    assert u & 0xFFFF == 0, "value is not bf16-exact"
    return u >> 16


def bf2f(h: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(h) & 0xFFFF) << 16))[0]


def golden_groups():
    with open(GOLDEN) as f:
        return json.load(f)["groups"]


def group_bits(g):
    x = np.zeros(32, np.uint16)
    for k, v in g["values"].items():
        x[int(k)] = f2bf(v)
    return x


def expected_codes(g):
    c = np.zeros(32, np.int64)
    for k, v in g["codes"].items():
        c[int(k)] = v
    return c


def unpack(codes_row):
    out = np.empty(codes_row.size * 2, np.int64)
    out[0::2] = codes_row & 0xF
    out[1::2] = codes_row >> 4
    return out


@pytest.mark.parametrize("g", golden_groups(), ids=lambda g: g["name"])
def test_hand_groups_oracle(g):
    x = group_bits(g)
    codes, scales = oracle.quant(x[None, :])
    assert scales[0, 0] == g["byte"]
    np.testing.assert_array_equal(unpack(codes[0]), expected_codes(g))
    for j, b in g.get("packed", {}).items():
        assert codes[0, int(j)] == b


@pytest.mark.parametrize("g", golden_groups(), ids=lambda g: g["name"])
def test_hand_groups_bruteforce(g):
    x = group_bits(g)
    codes, scales = bf.quant_rows([list(int(h) for h in x)])
    assert scales[0][0] == g["byte"]
    assert codes[0] == list(expected_codes(g))
    packed = bf.pack_codes(codes[0])
    for j, b in g.get("packed", {}).items():
        assert packed[int(j)] == b


def test_hand_groups_in_one_row():
    """All golden groups side by side in one row: group indexing and packing."""
    gs = golden_groups()
    row = np.concatenate([group_bits(g) for g in gs])
    codes, scales = oracle.quant(np.stack([row, row[::-1].copy()]))
    assert list(scales[0]) == [g["byte"] for g in gs]
    np.testing.assert_array_equal(unpack(codes[0]), np.concatenate([expected_codes(g) for g in gs]))


def all_finite_bf16_nonneg():
    h = np.arange(0, 0x7F80, dtype=np.uint32)
    return h


def test_encoder_every_bf16_below_8():
    """mxo_e2m1_code against the midpoint-table encoder for every bf16 q in [0, 8)."""
    mism = []
    for h in all_finite_bf16_nonneg():
        v = bf2f(h)
        if v >= 8.0:
            break
        a = oracle.e2m1_code(v)
        b = bf.e2m1_code(Fraction(v))
        if a != b:
            mism.append((v, a, b))
    assert not mism, mism[:10]


def test_encoder_fp32_sample_and_properties():
    rng = np.random.default_rng(7)
    qs = rng.uniform(0.0, 8.0, 20000).astype(np.float32)
    # every midpoint and its fp32 neighbours
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]
    extra = []
    for m in mids:
        m32 = np.float32(m)
        extra += [np.nextafter(m32, np.float32(0)), m32, np.nextafter(m32, np.float32(9))]
    qs = np.concatenate([qs, np.array(extra, np.float32)])
    codes = []
    for q in np.sort(qs):
        a = oracle.e2m1_code(float(q))
        assert a == bf.e2m1_code(Fraction(float(q))), float(q)
        codes.append(a)
    assert all(x <= y for x, y in zip(codes, codes[1:])), "encoder must be monotone"
    for c, v in enumerate(E2M1):
        assert oracle.e2m1_code(v) == c, "representable values map to themselves"
    assert oracle.e2m1_code(1e30) == 7


def test_scale_byte_every_bf16():
    """Scale byte from the fp32 bit rule against the rational formulation, every finite amax."""
    mism = []
    for h in all_finite_bf16_nonneg():
        v = bf2f(h)
        a = oracle.scale_byte(v)
        b = bf.scale_exponent(bf.bf16_bits_to_fraction(int(h))) + 127
        if a != b:
            mism.append((hex(int(h)), a, b))
    assert not mism, mism[:10]


def test_decode_table():
    for byte in (0, 1, 100, 125, 127, 128, 254):
        for code in range(16):
            want = bf.decode(code, byte)
            got = oracle.decode(code, byte)
            assert Fraction(got) == want
            if code == 8:
                assert np.signbit(got)


def test_invariants_random_groups():
    x = inputs.binade_spread(64, 32 * 64, seed=11, lo=-40, hi=40)
    xb = inputs.bits(x)
    codes, scales = oracle.quant(xb)
    assert scales.max() <= 254
    c = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(64, -1)
    mag = (c & 7).reshape(64, -1, 32)
    xf = x.float().numpy().reshape(64, -1, 32)
    nonzero = np.abs(xf).max(axis=2) > 0
    # (i) the largest code of every nonzero group is 4.0 or 6.0 (codes 6 / 7)
    assert np.all(np.isin(mag.max(axis=2)[nonzero], [6, 7]))
    # (iv) |x - deq(x)| <= 2^s elementwise
    deq = oracle.dequant(codes, scales).reshape(64, -1, 32)
    s = scales.astype(np.int64) - 127
    assert np.all(np.abs(xf - deq) <= np.ldexp(1.0, s)[..., None])
    # (ii) idempotence, signed zeros included
    deq_bits = inputs.bits(torch.from_numpy(deq.reshape(64, -1)).to(torch.bfloat16))
    codes2, scales2 = oracle.quant(deq_bits)
    np.testing.assert_array_equal(codes2, codes)
    np.testing.assert_array_equal(scales2, scales)


@pytest.mark.parametrize("case", ["randn", "binades", "tiny_and_huge"])
def test_bruteforce_gemm_4x64x64(case):
    M, N, K = 4, 64, 64
    if case == "randn":
        A, B = inputs.shape_inputs(M, N, K, seed=5)
    elif case == "binades":
        A = inputs.binade_spread(M, K, seed=6, lo=-12, hi=12)
        B = inputs.binade_spread(N, K, seed=7, lo=-12, hi=12)
    else:
        A = inputs.binade_spread(M, K, seed=8, lo=-130, hi=-110)
        B = inputs.binade_spread(N, K, seed=9, lo=100, hi=120)
    Ab, Bb = inputs.bits(A), inputs.bits(B)
    C = oracle.gemm(Ab, Bb)
    Cb, (ca, sa), (cb, sb) = bf.gemm([list(map(int, r)) for r in Ab], [list(map(int, r)) for r in Bb])
    codes_a, scales_a = oracle.quant(Ab)
    codes_b, scales_b = oracle.quant(Bb)
    assert [list(map(int, r)) for r in scales_a] == sa
    assert [list(map(int, r)) for r in scales_b] == sb
    assert [bf.pack_codes(r) for r in ca] == [list(map(int, r)) for r in codes_a]
    assert [bf.pack_codes(r) for r in cb] == [list(map(int, r)) for r in codes_b]
    assert [list(map(int, r)) for r in C] == Cb


def test_closed_form_all_ones():
    for K in (512, 1536, 2048, 7168):
        A = np.full((2, K), 0x3F80, np.uint16)
        B = np.full((3, K), 0x3F80, np.uint16)
        codes, scales = oracle.quant(A)
        assert np.all(codes == 0x66) and np.all(scales == 0x7D)
        C = oracle.gemm(A, B)
        assert np.all(C == f2bf(float(K)))


def test_closed_form_k32_hand_sums():
    a = np.zeros((2, 32), np.uint16)
    b = np.zeros((2, 32), np.uint16)
    # row 0: representable at s=0 -> exact: 4*3 + 2*(-1.5) + 1*6 + 0.5*2 = 16
    for k, v in enumerate([4.0, 2.0, 1.0, 0.5]):
        a[0, k] = f2bf(v)
    for k, v in enumerate([3.0, -1.5, 6.0, 2.0]):
        b[0, k] = f2bf(v)
    # row 1 of A: 5.0 ties to 4.0 and 2.5 ties to 2.0 (s=0); 0.3125 -> q 0.3125 -> 0.5
    for k, v in enumerate([5.0, 2.5, 0.3125]):
        a[1, k] = f2bf(v)
    # row 1 of B: amax 7 -> s=1: 7 -> 8, 3 -> q 1.5 -> 3, -0.75 -> q -0.375 -> -0.5 (dequant -1)
    for k, v in enumerate([7.0, 3.0, -0.75]):
        b[1, k] = f2bf(v)
    C = oracle.gemm(a, b)
    want = {(0, 0): 16.0,
            (0, 1): 4 * 8 + 2 * 3 + 1 * -1.0,
            (1, 0): 4 * 3 + 2 * -1.5 + 0.5 * 6,
            (1, 1): 4 * 8 + 2 * 3 + 0.5 * -1.0}
    for (m, n), v in want.items():
        assert C[m, n] == f2bf(v), (m, n, bf2f(C[m, n]), v)


def representable(rows, K, seed):
    """MXFP4-representable bf16 matrix: random codes and bytes, each group's
    largest magnitude code forced to 6 or 7, decoded with the e2m1 table."""
    rng = np.random.default_rng(seed)
    G = K // 32
    mag = rng.integers(0, 8, (rows, K))
    sign = rng.integers(0, 2, (rows, K))
    top = rng.integers(6, 8, (rows, G))
    pos = rng.integers(0, 32, (rows, G))
    for r in range(rows):
        for g in range(G):
            grp = mag[r, g * 32:(g + 1) * 32]
            np.minimum(grp, top[r, g], out=grp)
            grp[pos[r, g]] = top[r, g]
    codes = mag | (sign << 3)
    byte = rng.integers(120, 134, (rows, G))
    vals = np.array(E2M1)[mag] * np.ldexp(1.0, np.repeat(byte - 127, 32, axis=1))
    vals = np.where(sign == 1, -vals, vals)
    bits = inputs.bits(torch.from_numpy(vals).to(torch.bfloat16))
    return bits, codes, byte, vals


def test_closed_form_representable_is_textbook_matmul():
    M, N, K = 8, 24, 256
    Ab, ca, sa, Av = representable(M, K, 1)
    Bb, cb, sb, Bv = representable(N, K, 2)
    codes, scales = oracle.quant(Ab)
    np.testing.assert_array_equal(scales, sa)
    np.testing.assert_array_equal(unpack(codes.reshape(-1)).reshape(M, K), ca)
    ref = Av @ Bv.T                       # exact in fp64 for these magnitudes
    C = oracle.gemm(Ab, Bb)
    want = np.array([[bf.bf16_round(Fraction(float(v))) for v in row] for row in ref], np.uint16)
    np.testing.assert_array_equal(C, want)


@pytest.mark.parametrize("d,bits", [
    (1.0 + 2.0 ** -8, 0x3F80),            # tie -> even (down)
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),
    (1.0 + 3 * 2.0 ** -8, 0x3F82),        # tie -> even (up)
    (-(1.0 + 2.0 ** -8), 0xBF80),
    (2.0 ** -133, 0x0001),                # smallest bf16 subnormal
    (2.0 ** -134, 0x0000),                # tie -> even zero
    (0.75 * 2.0 ** -133, 0x0001),
    (-0.0, 0x8000),
    ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),
    ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),  # tie at the top rounds to infinity
    (3.0e38 * 2, 0x7F80),
])
def test_bf16_rounding_cases(d, bits):
    assert oracle.bf16_from_double(d) == bits
    if d != 0.0:                          # a Fraction has no signed zero
        assert bf.bf16_round(Fraction(d)) == bits


def test_bf16_rounding_random_against_exact():
    rng = np.random.default_rng(3)
    ds = rng.standard_normal(3000) * np.ldexp(1.0, rng.integers(-140, 120, 3000))
    for d in ds:
        assert oracle.bf16_from_double(float(d)) == bf.bf16_round(Fraction(float(d)))


def test_oracle_is_built_with_threads():
    assert oracle.num_threads() >= 1


# ---------------------------------------------------------------------------
# The a16wfp4 product (A unquantised bf16, B quantised): oracle.gemm_a16w4


def test_bf16_values_every_finite_pattern():
    """The exact widening of every finite bf16 pattern, against the rational
    decoding of the brute force."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    vals = oracle.bf16_values(bits)
    for h, v in zip(bits[finite][::97], vals[finite][::97]):
        assert Fraction(float(v)) == bf.bf16_bits_to_fraction(int(h)), hex(int(h))
    assert np.array_equal(np.signbit(vals[finite]), (bits[finite] & 0x8000) != 0)


@pytest.mark.parametrize("case", ["randn", "binades", "tiny_and_huge"])
def test_bruteforce_a16w4_4x64x64(case):
    M, N, K = 4, 64, 64
    if case == "randn":
        A, B = inputs.shape_inputs(M, N, K, seed=15)
    elif case == "binades":
        A = inputs.binade_spread(M, K, seed=16, lo=-12, hi=12)
        B = inputs.binade_spread(N, K, seed=17, lo=-12, hi=12)
    else:
        A = inputs.binade_spread(M, K, seed=18, lo=-120, hi=-100)
        B = inputs.binade_spread(N, K, seed=19, lo=90, hi=110)
    Ab, Bb = inputs.bits(A), inputs.bits(B)
    C = oracle.gemm_a16w4(Ab, Bb)
    Cb = bf.gemm_a16w4([list(map(int, r)) for r in Ab], [list(map(int, r)) for r in Bb])
    assert [list(map(int, r)) for r in C] == Cb


def test_a16w4_equals_a4w4_when_A_is_representable():
    """Quantisation is the identity on MXFP4-representable A, so both products agree."""
    M, N, K = 8, 40, 256
    Ab, _, _, _ = representable(M, K, 5)
    B = inputs.binade_spread(N, K, seed=21, lo=-8, hi=8)
    Bb = inputs.bits(B)
    np.testing.assert_array_equal(oracle.gemm_a16w4(Ab, Bb), oracle.gemm(Ab, Bb))


def test_a16w4_differs_from_a4w4_on_general_A():
    """On N(0,1) activations the two products are different functions (the
    activation's quantisation error is not in a16w4)."""
    A, B = inputs.shape_inputs(8, 64, 512, seed=22)
    Ab, Bb = inputs.bits(A), inputs.bits(B)
    assert np.mean(oracle.gemm_a16w4(Ab, Bb) != oracle.gemm(Ab, Bb)) > 0.5


def test_a16w4_closed_form_representable_B_is_textbook_matmul():
    """With B representable, dequant(quant(B)) = B and the product is the
    textbook matmul of the two bf16 matrices, rounded once (the fp64 sum is
    exact at these magnitudes: 11-bit products over ~30 binades)."""
    M, N, K = 6, 24, 256
    A, _ = inputs.shape_inputs(M, 8, K, seed=23)
    Ab = inputs.bits(A)
    Bb, _, _, Bv = representable(N, K, 24)
    ref = A.float().double().numpy() @ Bv.T
    want = np.array([[bf.bf16_round(Fraction(float(v))) for v in row] for row in ref], np.uint16)
    np.testing.assert_array_equal(oracle.gemm_a16w4(Ab, Bb), want)


def test_a16w4_all_ones():
    for K in (512, 7168):
        A = np.full((2, K), 0x3F80, np.uint16)
        B = np.full((3, K), 0x3F80, np.uint16)
        assert np.all(oracle.gemm_a16w4(A, B) == oracle.bf16_from_double(float(K)))


def _bitlevel_e2m1(q32: np.ndarray) -> np.ndarray:
    """A second e2m1 encoder, vectorised and independent of the oracle: the
    bit-level method of the kernelindex.com amd-mxfp4-mm pages (submission
    755056, section "Software MXFP4 quant"), written out from its idea.
    For |q| >= 6 the code saturates at 7.  Below 1 the fp32 adder does the
    rounding: adding 2^22 leaves a sum whose ulp is 0.5, so the hardware's
    round-to-nearest-even puts |q| on the e2m1 subnormal grid {0, 0.5, 1},
    and the sum's bit pattern minus that of 2^22 counts the halves.  From 1
    to 6 the code is the fp32 pattern with the exponent rebased from 127 to
    e2m1's bias 1 and the 22 low significand bits dropped by an integer
    round-half-to-even (add 2^21 - 1 plus the kept low bit, then shift).
    The sign bit of q becomes bit 3 of the code."""
    u = q32.view(np.uint32)
    sign = (u >> 31).astype(np.uint32)
    a = (u & np.uint32(0x7FFFFFFF)).view(np.float32)
    au = a.view(np.uint32)
    with np.errstate(over="ignore"):
        small = ((a + np.float32(4194304.0)).view(np.uint32) - np.float32(4194304.0).view(np.uint32)) & 0xFF
    keep = (au >> 22) & 1
    normal = ((au - np.uint32(126 << 23) + np.uint32((1 << 21) - 1) + keep) >> 22) & 0xFF
    code = np.where(a >= np.float32(6.0), 7, np.where(a < np.float32(1.0), small, normal)).astype(np.uint32)
    return (code | (sign << 3)).astype(np.int64)


def test_encoder_matches_the_pages_bit_level_method():
    """oracle.e2m1_code against the pages' bit-level encoder (fp32 adder
    rounding below 1, integer round-half-even above) for every bf16 q in
    [0, 8) of both signs, and for every fp32 q in [0, 8) on a 2^-14 grid
    plus the neighbours of each tie point."""
    h = np.arange(0, 0x4100, dtype=np.uint32)            # bf16 0 .. 8 (0x4100 = 8.0)
    pos = (h << 16).view(np.float32)
    qs = [pos, -pos, np.arange(0, 8 * 16384, dtype=np.float64).astype(np.float32) / np.float32(16384)]
    for m in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0):
        m32 = np.float32(m)
        qs.append(np.array([np.nextafter(m32, np.float32(0)), m32, np.nextafter(m32, np.float32(9))], np.float32))
    q = np.concatenate(qs).astype(np.float32)
    ref = _bitlevel_e2m1(q)
    got = np.array([oracle.e2m1_code(abs(float(v))) | (8 if np.signbit(v) else 0) for v in q], np.int64)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(q[i]), int(got[i]), int(ref[i])) for i in bad[:10]]


@pytest.mark.parametrize("byte", [0, 1, 2, 100, 125, 126, 127, 128, 200, 253])
def test_quant_matches_the_pages_bit_level_method(byte):
    """oracle.quant against the bit-level encoder on whole groups: every
    finite bf16 value whose group scale is 2^(byte - 127) sits in a group
    next to an element that fixes that scale; the codes must equal the
    bit-level encoding of x * 2^-s (exact in fp32 here)."""
    s = byte - 127
    # R = 2^(s+2) gives this scale byte; at byte 253 (the largest a finite
    # input reaches) the largest finite bf16 rounds up to R = 2^128
    amax = np.ldexp(1.0, s + 2) if byte < 253 else float((np.uint32(0x7F7F) << 16).view(np.float32))
    h = np.arange(0, 0x7F80, dtype=np.uint32)
    xs = (h << 16).view(np.float32).astype(np.float64)
    keep = (xs <= amax) & (xs * np.ldexp(1.0, -s) >= np.ldexp(1.0, -120))   # no fp32 underflow in q
    if byte <= 2:
        keep = xs <= amax
    xs = np.concatenate([xs[keep], -xs[keep]])
    x_b = (xs.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    n = x_b.size
    rows = (n + 30) // 31
    grid = np.zeros((rows, 32), np.uint16)
    flat = np.zeros(rows * 31, np.uint16)
    flat[:n] = x_b
    grid[:, 1:] = flat.reshape(rows, 31)
    grid[:, 0] = np.uint16(np.float32(amax).view(np.uint32) >> 16)
    codes, scales = oracle.quant(grid)
    assert (scales[:, 0] == byte).all()
    got = np.empty((rows, 32), np.int64)
    got[:, 0::2] = codes & 0xF
    got[:, 1::2] = codes >> 4
    got = got[:, 1:].reshape(-1)[:n]
    q = (xs * np.ldexp(1.0, -max(s, -127))).astype(np.float32)
    if byte == 0:
        q = (xs * np.ldexp(1.0, 127)).astype(np.float32)
    np.testing.assert_array_equal(got, _bitlevel_e2m1(q))
