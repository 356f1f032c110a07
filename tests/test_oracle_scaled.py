"""Pins of the oracle's scaled epilogue (CPU only).

The scaled entry points define D[m][n] = out(((float)C[m][n] * scale_a[m]) *
scale_b[n]) with binary32 roundings to nearest even and a nearest-even
conversion to the output format (the tutorial's gemm_blockscaled with one K
block).  The oracle implements it in C; these tests pin it against
hand-worked roundings, numpy's binary16 conversion, the nearest-even
property checked by brute force over the neighbours, exact rational
arithmetic, and closed forms (unit and power-of-two scales, sign symmetry).
"""
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from precision_integer_gemm_amd.inputs import scale_vector

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rounding_worked.txt")
FMT = {"f32": oracle.FMT_F32, "bf16": oracle.FMT_BF16, "f16": oracle.FMT_F16}


def one(x, fmt):
    """Round one binary32 value through the epilogue (unit scales)."""
    # C must be an integer; feed x through a scale instead: C = 1, scale_a = x.
    out = oracle.scaled_epilogue(np.array([[1]], np.int32), np.array([x], np.float32),
                                 np.array([1.0], np.float32), fmt)
    return out[0, 0]


def test_hand_worked_roundings():
    n = 0
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            fmt, x, want = line.split()[:3]
            assert np.float32(float(x)) == float(x), "golden inputs are binary32 values"
            got = one(float(x), FMT[fmt])
            assert got == float(want), (fmt, x, got, want)
            n += 1
    assert n >= 15


def test_f16_matches_numpy_conversion():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * np.float32(1000.0),
        (rng.standard_normal(4000) * 1e-5).astype(np.float32),   # subnormal range
        (rng.standard_normal(2000) * 6e4).astype(np.float32),    # near overflow
        np.array([65504, 65519, 65520, 65536, -65520, 0.0, -0.0], np.float32)])
    C = np.ones((1, len(x)), np.int32)
    got = oracle.scaled_epilogue(C, np.ones(1, np.float32), x, oracle.FMT_F16)[0]
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def _f32(v: float) -> float:
    return struct.unpack("<f", struct.pack("<f", v))[0]


def _bf16_neighbours(x: float):
    """bfloat16 values just below and above |x| (truncation and the next up)."""
    bits = struct.unpack("<I", struct.pack("<f", abs(x)))[0]
    lo = bits & 0xFFFF0000
    hi = lo + 0x10000
    as_val = lambda b: Fraction(struct.unpack("<f", struct.pack("<I", b))[0]) if b < 0x7F800000 \
        else Fraction(2) ** 128
    return lo, hi, as_val(lo), as_val(hi)


def test_bf16_is_nearest_even_by_brute_force():
    rng = np.random.default_rng(12)
    raw = rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32)
    x = raw.view(np.float32)
    x = x[np.isfinite(x)]
    C = np.ones((1, len(x)), np.int32)
    got = oracle.scaled_epilogue(C, np.ones(1, np.float32), x, oracle.FMT_BF16)[0]
    for xi, gi in zip(x[:4000], got[:4000]):
        xf = Fraction(float(xi))
        lo, hi, vlo, vhi = _bf16_neighbours(float(xi))
        dlo, dhi = abs(xf) - vlo, vhi - abs(xf)
        if dlo < dhi or (dlo == dhi and (lo >> 16) % 2 == 0):
            want = vlo
        else:
            want = vhi
        want = float(want) if want != Fraction(2) ** 128 else float("inf")
        want = -want if xi < 0 else want
        assert gi == want, (float(xi), gi, want)


def test_multiply_order_against_exact_arithmetic():
    rng = np.random.default_rng(13)
    C = rng.integers(-2**20, 2**20, (8, 16)).astype(np.int32)
    sa = scale_vector(21, 0, 8)
    sb = scale_vector(21, 1, 16)
    got = oracle.scaled_epilogue(C, sa, sb, oracle.FMT_F32)
    for m in range(8):
        for n in range(16):
            t = _f32(float(C[m, n]))                        # int -> binary32
            y = _f32(float(Fraction(t) * Fraction(float(sa[m]))))
            z = _f32(float(Fraction(y) * Fraction(float(sb[n]))))
            assert got[m, n] == z


def test_order_matters_somewhere():
    # (t * sa) * sb and t * (sa * sb) differ for some inputs, so the pin above
    # does fix the order the definition states.
    rng = np.random.default_rng(14)
    t = rng.integers(-2**20, 2**20, 20000).astype(np.float32)
    sa = scale_vector(22, 0, 20000)
    sb = scale_vector(22, 1, 20000)
    left = (t * sa) * sb
    right = t * (sa * sb)
    assert np.any(left != right)


@pytest.mark.parametrize("fmt", [oracle.FMT_F32, oracle.FMT_BF16, oracle.FMT_F16])
def test_unit_scales_give_the_integer(fmt):
    C = np.array([[0, 1, -7, 255, -2048]], np.int32)  # exact in every format
    got = oracle.scaled_epilogue(C, np.ones(1, np.float32), np.ones(5, np.float32), fmt)
    assert np.array_equal(got, C.astype(np.float64))


def test_power_of_two_scales_are_exact():
    rng = np.random.default_rng(15)
    C = rng.integers(-2**23, 2**23, (6, 9)).astype(np.int32)
    ea = rng.integers(-20, 20, 6)
    eb = rng.integers(-20, 20, 9)
    got = oracle.scaled_epilogue(C, np.ldexp(1.0, ea).astype(np.float32),
                                 np.ldexp(1.0, eb).astype(np.float32), oracle.FMT_F32)
    want = C.astype(np.float64) * np.ldexp(1.0, ea)[:, None] * np.ldexp(1.0, eb)[None, :]
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fmt", [oracle.FMT_F32, oracle.FMT_BF16, oracle.FMT_F16])
def test_sign_symmetry(fmt):
    rng = np.random.default_rng(16)
    C = rng.integers(-5000, 5000, (5, 7)).astype(np.int32)
    sa, sb = scale_vector(23, 0, 5), scale_vector(23, 1, 7)
    a = oracle.scaled_epilogue(C, sa, sb, fmt)
    b = oracle.scaled_epilogue(C, -sa, sb, fmt)
    c = oracle.scaled_epilogue(-C, sa, -sb, fmt)
    assert np.array_equal(a, -b) and np.array_equal(a, c)


def test_gemm_scaled_composes_the_exact_product():
    from precision_integer_gemm_amd.inputs import custom_operands
    A, B = custom_operands("w4a8", 9, 13, 96, seed=5)
    sa, sb = scale_vector(5, 0, 9), scale_vector(5, 1, 13)
    C = oracle.gemm_w4a8(A, B, 9, 13, 96)
    assert np.array_equal(oracle.gemm_scaled("w4a8", A, B, sa, sb, 9, 13, 96, oracle.FMT_BF16),
                          oracle.scaled_epilogue(C, sa, sb, oracle.FMT_BF16))
