"""Mutation tests of the oracle's pins (CPU only).

Each case plants one plausible mistake into a copy of oracle/mxoracle.c (a
wrong rounding constant or exponent offset, a dropped clamp, sign or term,
ties going the wrong way, swapped nibbles or operands, truncating instead of
rounding), builds it, and runs tests/test_oracle.py against it in a fresh
process: at least one pin must fail.  The unmodified copy must pass.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "mxoracle.c")

# (name, text in mxoracle.c, replacement)
MUTANTS = [
    ("amax_rounding_constant", "+ 0x00200000u", "+ 0x00100000u"),
    ("amax_not_rounded_up", "+ 0x00200000u", "+ 0x0u"),
    ("exponent_offset", "int s = e - 129;", "int s = e - 128;"),
    ("no_low_clamp", "if (s < -127) s = -127;", ""),
    ("ties_to_odd", "(c & 1) == 0 && (best & 1) == 1", "(c & 1) == 1 && (best & 1) == 0"),
    ("saturate_too_early", "if (q >= 6.0) return 7;", "if (q >= 5.0) return 7;"),
    ("sign_dropped", "if (h & 0x8000u) code |= 8;", ""),
    ("nibbles_swapped", "(uint8_t)(nib[0] | (nib[1] << 4))", "(uint8_t)(nib[1] | (nib[0] << 4))"),
    ("scale_applied_backwards", "ldexp((double)bf16_to_float(h), -s)", "ldexp((double)bf16_to_float(h), s)"),
    ("decode_bias", "ldexp(kE2M1[code & 7], byte - 127)", "ldexp(kE2M1[code & 7], byte - 128)"),
    ("dequant_nibble_order", "(k & 1) ? (b >> 4) : (b & 0xF)", "(k & 1) ? (b & 0xF) : (b >> 4)"),
    ("gemm_dropped_term", "for (int k = 0; k < K; ++k) acc", "for (int k = 1; k < K; ++k) acc"),
    ("gemm_wrong_index", "acc += a[k] * b[k];", "acc += a[k] * b[K - 1 - k];"),
    ("bf16_truncates", "nearbyint(a / quantum)", "floor(a / quantum)"),
    ("bf16_no_subnormals", "if (e < -126) e = -126;", ""),
    ("amax_half_group", "if (v > amax) amax = v;", "if (v > amax && i < 16) amax = v;"),
    ("a16w4_sign_lost", "out[i] = (double)bf16_to_float(x[i]);", "out[i] = (double)bf16_to_float(x[i] & 0x7FFF);"),
]


def build_variant(tmp_path, name, old, new):
    src = open(SRC).read()
    if old is not None:
        assert src.count(old) == 1, "mutation target not unique or missing: %r" % old
        src = src.replace(old, new)
    c = tmp_path / ("%s.c" % name)
    c.write_text(src)
    so = tmp_path / ("%s.so" % name)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", str(c), "-o", str(so), "-lm"])
    return str(so)


def run_pins(lib):
    env = dict(os.environ, MX_ORACLE_LIB=lib, OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_oracle.py"), "-x", "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def test_unmodified_copy_passes_the_pins(tmp_path):
    rc, out = run_pins(build_variant(tmp_path, "original", None, None))
    assert rc == 0, out


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    rc, out = run_pins(build_variant(tmp_path, name, old, new))
    assert rc != 0, "mutant %s survived every pin:\n%s" % (name, out)
