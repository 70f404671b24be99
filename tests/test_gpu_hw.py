"""The gfx950 instructions the path rests on, checked directly on one wave
(libmx4hw.so, include/mx4_hwcheck.h; needs an MI355X).

* v_cvt_scalef32_pk_fp4_bf16, as the quantisers call it: every finite bf16
  input under the scale operand of every scale byte 0..254, against the
  oracle's e2m1 encoder of x * 2^-s (round to nearest even, saturation at 6,
  sign kept) -- the MXFP4 rule of the kernelindex.com amd-mxfp4-mm pages
  (submission 755056, "Software MXFP4 quant");
* v_cvt_scalef32_pk_bf16_fp4, as the a16wfp4 product widens its weight:
  every code under every scale byte against the oracle's decode;
* v_mfma_scale_f32_32x32x64_f8f6f4 with both operands e2m1: lane layout of
  the fragments, of the scale registers (only the low byte counts) and of
  the accumulators, against a host model of the block-scaled product.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
HWLIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "microscaled_mxfp4_block_amd",
                     "libmx4hw.so")
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def hw():
    if not os.path.exists(HWLIB):
        raise ImportError("libmx4hw.so is not built; run `python -m microscaled_mxfp4_block_amd.build`")
    L = ctypes.CDLL(HWLIB)
    P, I = ctypes.c_void_p, ctypes.c_int
    L.mxhw_cvt_fp4.argtypes = [P, I, I, P, P]
    L.mxhw_widen_fp4.argtypes = [I, P, P]
    L.mxhw_mfma_fp4.argtypes = [P, P, P, P, P, P]
    return L


def stream():
    return torch.cuda.current_stream().cuda_stream


def test_fp4_convert_every_finite_bf16_every_scale_byte():
    h = np.arange(0x10000, dtype=np.uint32)
    finite = h[((h >> 7) & 0xFF) != 0xFF]
    n = (finite.size + 7) // 8 * 8
    x = np.zeros(n, np.uint16)
    x[:finite.size] = finite
    nbytes = 255
    xd = torch.from_numpy(x.view(np.int16)).to(DEV)
    out = torch.empty(nbytes * n // 2, dtype=torch.uint8, device=DEV)
    assert hw().mxhw_cvt_fp4(xd.data_ptr(), n, nbytes, out.data_ptr(), stream()) == 0
    torch.cuda.synchronize()
    packed = out.cpu().numpy().reshape(nbytes, n // 2)
    got = np.empty((nbytes, n), np.uint8)
    got[:, 0::2] = packed & 0xF
    got[:, 1::2] = packed >> 4
    # the oracle's encoder on every bf16 magnitude below 8 (0x4100 = 8.0)
    table = np.array([oracle.e2m1_code(float((np.uint32(t) << 16).view(np.float32))) for t in range(0x4100)],
                     np.uint8)
    xs = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    mag = np.abs(xs)
    sign = ((x >> 15) & 1).astype(np.uint8) << 3
    for b in range(nbytes):
        s = max(b - 127, -127)
        q = mag * np.ldexp(1.0, -s)                      # exact in fp64
        big = q >= 8.0
        tiny = q < np.ldexp(1.0, -126)                    # far below the first rounding point 0.25
        qb = (np.where(big | tiny, 0.0, q).astype(np.float32).view(np.uint32) >> 16).astype(np.int64)
        code = np.where(big, 7, np.where(tiny, 0, table[np.minimum(qb, 0x40FF)])).astype(np.uint8)
        want = code | sign
        bad = np.nonzero(got[b] != want)[0]
        assert bad.size == 0, "byte %d: %d mismatches, e.g. %s" % (
            b, bad.size, [(hex(int(x[i])), int(got[b, i]), int(want[i])) for i in bad[:5]])


def test_fp4_widen_every_code_every_scale_byte():
    nbytes = 255
    out = torch.empty(nbytes * 16, dtype=torch.int16, device=DEV)
    assert hw().mxhw_widen_fp4(nbytes, out.data_ptr(), stream()) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16).reshape(nbytes, 16)
    checked = 0
    for b in range(nbytes):
        for c in range(16):
            v = oracle.decode(c, b)
            if abs(v) >= 2.0 ** 128:                     # past bf16's range: outside the contract
                continue
            f = np.float32(v)
            assert float(f) == v and (f.view(np.uint32) & 0xFFFF) == 0
            assert got[b, c] == (f.view(np.uint32) >> 16), (b, c, hex(int(got[b, c])), v)
            checked += 1
    assert checked == nbytes * 16 - 12   # 2^128 and above: codes 4, 6 at byte 253; 2, 3, 4, 6 at 254


def mfma_model(a, b, sa, sb):
    """Host model of one 32x32x64 block-scaled fp4 MFMA: lane L's fragment
    holds row L % 32, K elements 32 (L / 32) .. + 31 (element j in nibble j:
    byte j / 2, low nibble for even j) of its operand, scaled by
    2^(low byte of its scale word - 127); lane L's accumulator element e is
    output row 8 (e / 4) + 4 (L / 32) + e % 4 (a row of the first operand)
    and column L % 32 (a row of the second operand)."""
    def values(frag, sc):
        v = np.zeros((32, 64))
        for L in range(64):
            r, h = L % 32, L // 32
            scale = np.ldexp(1.0, int(sc[L] & 0xFF) - 127)
            for j in range(32):
                byte = frag[16 * L + j // 2]
                code = (byte >> (4 * (j % 2))) & 0xF
                v[r, 32 * h + j] = (-1.0 if code & 8 else 1.0) * E2M1[code & 7] * scale
        return v
    va, vb = values(a, sa), values(b, sb)
    d = va @ vb.T                                          # [row of a, row of b], exact in fp64 here
    out = np.zeros((64, 16))
    for L in range(64):
        for e in range(16):
            out[L, e] = d[8 * (e // 4) + 4 * (L // 32) + e % 4, L % 32]
    return out


@pytest.mark.parametrize("case", ["dense_near_one", "one_group_wide_scales", "sparse"])
def test_scaled_mfma_lane_layout(case):
    rng = np.random.default_rng({"dense_near_one": 1, "one_group_wide_scales": 2, "sparse": 3}[case])
    a = rng.integers(0, 256, 1024, dtype=np.uint8)
    b = rng.integers(0, 256, 1024, dtype=np.uint8)
    junk_a = rng.integers(0, 1 << 24, 64, dtype=np.uint32) << 8   # upper bytes of the scale words
    junk_b = rng.integers(0, 1 << 24, 64, dtype=np.uint32) << 8
    if case == "dense_near_one":
        sa = rng.integers(125, 130, 64, dtype=np.uint32)
        sb = rng.integers(125, 130, 64, dtype=np.uint32)
    elif case == "one_group_wide_scales":
        # only the first K group carries codes, so each output sums 32
        # products under one pair of scales; the pair spans a wide range
        a[512:] = 0
        b[512:] = 0
        sa = rng.integers(67, 188, 64, dtype=np.uint32)
        sb = rng.integers(67, 188, 64, dtype=np.uint32)
    else:
        a[rng.random(1024) < 0.8] = 0
        b[rng.random(1024) < 0.8] = 0
        sa = rng.integers(124, 131, 64, dtype=np.uint32)
        sb = rng.integers(124, 131, 64, dtype=np.uint32)
    want = mfma_model(a, b, sa, sb)
    assert np.array_equal(want.astype(np.float32).astype(np.float64), want), "model result not exact in fp32"
    t = lambda arr: torch.from_numpy(arr.view(np.int32) if arr.dtype == np.uint32 else arr).to(DEV)
    ad, bd = t(a), t(b)
    sad, sbd = t((sa | junk_a).astype(np.uint32)), t((sb | junk_b).astype(np.uint32))
    out = torch.empty(1024, dtype=torch.float32, device=DEV)
    assert hw().mxhw_mfma_fp4(ad.data_ptr(), bd.data_ptr(), sad.data_ptr(), sbd.data_ptr(), out.data_ptr(),
                              stream()) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64).reshape(64, 16)
    bad = np.argwhere(got != want)
    assert bad.size == 0, [(tuple(i), got[tuple(i)], want[tuple(i)]) for i in bad[:5]]
