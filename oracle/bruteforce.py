"""Exact pure-Python MXFP4 brute force -- TEST INFRASTRUCTURE ONLY.

A second, separately written implementation of the same method, used to pin
the C oracle on tiny inputs (4x64x64 and the like).  It is deliberately
formulated differently from ``mxoracle.c``:

* the power-of-two rounding of the group maximum is written as plain
  arithmetic on rationals: with amax = f * 2^e, f in [1, 2), the rounded
  value is 2^(e+1) when f >= 7/4 and 2^e otherwise (this is what adding
  0x00200000 to the fp32 bits and masking off the significand does in the
  "Software MXFP4 quant" section of kernelindex.com amd-mxfp4-mm submission
  755056); s = clamp(log2(rounded) - 2, -127, 127), byte = s + 127;
* e2m1 rounding is a table lookup over the seven decision midpoints
  {1/4, 3/4, 5/4, 7/4, 5/2, 7/2, 5} with the tie going to the even code;
* every value is a ``fractions.Fraction``: the GEMM sum is exact and the
  bf16 rounding is done by exact integer arithmetic.

Slow by design: use it only on a few thousand elements.
"""
from __future__ import annotations

from fractions import Fraction
import struct

E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
        Fraction(2), Fraction(3), Fraction(4), Fraction(6)]
# Decision midpoints between consecutive e2m1 magnitudes.
MIDPOINTS = [(E2M1[i] + E2M1[i + 1]) / 2 for i in range(7)]


def bf16_bits_to_fraction(h: int) -> Fraction:
    """Exact value of a (finite) bf16 bit pattern."""
    sign = -1 if h & 0x8000 else 1
    exp = (h >> 7) & 0xFF
    man = h & 0x7F
    if exp == 0xFF:
        raise ValueError("non-finite bf16 outside the contract")
    if exp == 0:
        mag = Fraction(man, 128) * Fraction(2) ** -126
    else:
        mag = (1 + Fraction(man, 128)) * Fraction(2) ** (exp - 127)
    return sign * mag


def _floor_log2(x: Fraction) -> int:
    """e with 2^e <= x < 2^(e+1), for x > 0, exactly."""
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    elif Fraction(2) ** (e + 1) <= x:
        e += 1
    return e


def scale_exponent(amax: Fraction) -> int:
    """s for a group whose largest magnitude is amax (>= 0)."""
    if amax == 0:
        return -127
    e = _floor_log2(amax)
    f = amax / Fraction(2) ** e
    e_r = e + 1 if f >= Fraction(7, 4) else e
    return max(-127, min(127, e_r - 2))


def e2m1_code(q: Fraction) -> int:
    """Magnitude code of |q| (q >= 0): midpoint table, ties to the even code."""
    code = 0
    for i, mid in enumerate(MIDPOINTS):
        if q > mid or (q == mid and (i + 1) % 2 == 0):
            code = i + 1
    return code


def quant_rows(x_bits):
    """x_bits: list of rows of bf16 ints.  Returns (codes, bytes) per row, codes
    as lists of 4-bit ints in k order, bytes as lists per group."""
    codes, scales = [], []
    for row in x_bits:
        K = len(row)
        assert K % 32 == 0
        rc, rs = [], []
        for g in range(K // 32):
            grp = row[32 * g:32 * g + 32]
            vals = [bf16_bits_to_fraction(h) for h in grp]
            s = scale_exponent(max(abs(v) for v in vals))
            rs.append(s + 127)
            for h, v in zip(grp, vals):
                c = e2m1_code(abs(v) / Fraction(2) ** s)
                if h & 0x8000:
                    c |= 8
                rc.append(c)
        codes.append(rc)
        scales.append(rs)
    return codes, scales


def pack_codes(codes_row):
    """k-ordered 4-bit codes -> bytes, even k in the low nibble."""
    return [codes_row[2 * j] | (codes_row[2 * j + 1] << 4) for j in range(len(codes_row) // 2)]


def decode(code: int, byte: int) -> Fraction:
    v = E2M1[code & 7] * Fraction(2) ** (byte - 127)
    return -v if code & 8 else v


def bf16_round(x: Fraction) -> int:
    """Exact round-to-nearest-even of a rational to bf16 bits."""
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    if a == 0:
        return sign
    e = max(_floor_log2(a), -126)
    quantum = Fraction(2) ** (e - 7)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if r > (2 - Fraction(1, 128)) * Fraction(2) ** 127:
        return sign | 0x7F80
    f32 = struct.unpack("<I", struct.pack("<f", float(r)))[0]   # r is exactly representable
    return sign | (f32 >> 16)


def gemm_a16w4(A_bits, B_bits):
    """C = bf16(exact sum_k A[m,k] deqB[n,k]) with A's bf16 values unquantised."""
    cb, sb = quant_rows(B_bits)
    K = len(A_bits[0])
    Av = [[bf16_bits_to_fraction(a) for a in row] for row in A_bits]
    Bd = [[decode(cb[n][k], sb[n][k // 32]) for k in range(K)] for n in range(len(B_bits))]
    return [[bf16_round(sum((a * b for a, b in zip(Av[m], Bd[n])), Fraction(0))) for n in range(len(Bd))]
            for m in range(len(Av))]


def gemm(A_bits, B_bits):
    """C = bf16(exact sum_k deqA[m,k] deqB[n,k]); A_bits [M][K], B_bits [N][K]."""
    ca, sa = quant_rows(A_bits)
    cb, sb = quant_rows(B_bits)
    K = len(A_bits[0])
    Ad = [[decode(ca[m][k], sa[m][k // 32]) for k in range(K)] for m in range(len(A_bits))]
    Bd = [[decode(cb[n][k], sb[n][k // 32]) for k in range(K)] for n in range(len(B_bits))]
    C = []
    for m in range(len(Ad)):
        C.append([bf16_round(sum((a * b for a, b in zip(Ad[m], Bd[n])), Fraction(0)))
                  for n in range(len(Bd))])
    return C, (ca, sa), (cb, sb)
