"""Pins of the oracle's fp8 GEMM with e5m2 operands: decode, encode, product.

The decode is checked against PyTorch's float8_e5m2 (an independent
implementation of the same OCP format) on all 256 codes and against values the
definition fixes; the encode against PyTorch's nearest-even conversion on every
midpoint and on random values inside the finite range, and against the
IEEE-style overflow to infinity by hand; the product against exact rational
arithmetic on small shapes, across the whole exponent range (which no double
sum holds exactly), and closed forms.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from precision_integer_gemm_amd.inputs import random_bytes

torch = pytest.importorskip("torch")

ALL = np.arange(256, dtype=np.uint8)


def torch_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e5m2).to(torch.float64).numpy()


def torch_encode(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e5m2).view(torch.uint8).numpy()


def test_decode_matches_torch_on_every_code():
    got, want = oracle.fp8_e5m2_decode(ALL), torch_decode(ALL)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


@pytest.mark.parametrize("code,value", [
    (0x3C, 1.0), (0x40, 2.0), (0x3F, 1.75), (0x7B, 57344.0), (0xFB, -57344.0),
    (0x04, 2.0 ** -14), (0x01, 2.0 ** -16), (0x03, 3 * 2.0 ** -16), (0x00, 0.0),
    (0x7C, math.inf), (0xFC, -math.inf),
])
def test_decode_definition_values(code, value):
    assert oracle.fp8_e5m2_decode(np.array([code], np.uint8))[0] == value


def test_decode_nan_codes():
    v = oracle.fp8_e5m2_decode(np.array([0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF], np.uint8))
    assert np.isnan(v).all()


def test_encode_round_trips_every_finite_code():
    finite = ALL[np.isfinite(torch_decode(ALL))]
    assert np.array_equal(oracle.fp8_e5m2_encode(oracle.fp8_e5m2_decode(finite)), finite)


def test_encode_midpoints_and_random_values_match_torch():
    vals = np.sort(np.unique(torch_decode(ALL)[np.isfinite(torch_decode(ALL))]))
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(9)
    rand = rng.uniform(-60000.0, 60000.0, 20000).astype(np.float32).astype(np.float64)
    small = rng.uniform(-2.0 ** -12, 2.0 ** -12, 5000).astype(np.float32).astype(np.float64)
    for x in (mids, rand, small):
        assert np.array_equal(oracle.fp8_e5m2_encode(x), torch_encode(x))


def test_encode_overflow_to_infinity_by_hand():
    # the largest finite value is 57344; the next binade would start at 65536;
    # the midpoint 61440 ties to the even neighbour, 65536, which is infinity
    x = np.array([57344.0, 61439.0, 61440.0, 1e6, math.inf, -61440.0, -math.inf, 58000.0])
    assert oracle.fp8_e5m2_encode(x).tolist() == [0x7B, 0x7B, 0x7C, 0x7C, 0x7C, 0xFC, 0xFC, 0x7B]
    assert oracle.fp8_e5m2_encode(np.array([math.nan]))[0] & 0x7F == 0x7F
    # ties to even below: 1.125 lies between 1.0 (0x3C) and 1.25 (0x3D) -> 0x3C
    assert oracle.fp8_e5m2_encode(np.array([1.125, 1.375]))[0] == 0x3C
    assert oracle.fp8_e5m2_encode(np.array([1.375]))[0] == 0x3E


def finite_codes(stream, n):
    c = random_bytes(stream, n)
    return np.where((c & 0x7C) == 0x7C, c & 0xFB, c).astype(np.uint8)   # no inf / NaN


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (2, 3, 5), (4, 3, 16), (3, 5, 33)])
def test_gemm_matches_exact_rational_brute_force(M, N, K):
    A = finite_codes(300 + M, M * K).reshape(M, K)
    B = finite_codes(400 + N, N * K).reshape(N, K)
    C, Cabs = oracle.gemm_fp8_e5m2(A, B, M, N, K)
    da = [[Fraction(v) for v in row] for row in torch_decode(A)]
    db = [[Fraction(v) for v in row] for row in torch_decode(B)]
    for m in range(M):
        for n in range(N):
            s = sum(da[m][k] * db[n][k] for k in range(K))
            sa = sum(abs(da[m][k] * db[n][k]) for k in range(K))
            # the nearest double of the exact sums
            assert C[m, n] == float(s) and Cabs[m, n] == float(sa)


def test_gemm_exact_across_the_exponent_range():
    # 57344^2 + 2^-32 - 57344^2 + 2^-32: a double sum in k order loses both
    # small terms; the exact sum is 2^-31
    a = np.array([[57344.0, 2.0 ** -16, -57344.0, 2.0 ** -16]])
    b = np.array([[57344.0, 2.0 ** -16, 57344.0, 2.0 ** -16]])
    A, B = oracle.fp8_e5m2_encode(a).reshape(1, 4), oracle.fp8_e5m2_encode(b).reshape(1, 4)
    C, Cabs = oracle.gemm_fp8_e5m2(A, B, 1, 1, 4)
    assert C[0, 0] == 2.0 ** -31
    assert Cabs[0, 0] == 2 * 57344.0 ** 2 + 2.0 ** -31


def test_gemm_closed_forms_and_nonfinite():
    K = 4096
    ones = np.full((3, K), 0x3C, np.uint8)
    C, Cabs = oracle.gemm_fp8_e5m2(ones, ones[:2], 3, 2, K)
    assert (C == K).all() and (Cabs == K).all()
    big, nbig = np.full((2, K), 0x7B, np.uint8), np.full((2, K), 0xFB, np.uint8)
    C, _ = oracle.gemm_fp8_e5m2(big, nbig, 2, 2, K)
    assert (C == -(57344.0 ** 2) * K).all()
    A = np.full((3, 8), 0x3C, np.uint8)
    A[1, 3] = 0x7C                                                   # +inf
    A[2, 5] = 0x7E                                                   # NaN
    C, _ = oracle.gemm_fp8_e5m2(A, np.full((2, 8), 0x3C, np.uint8), 3, 2, 8)
    assert (C[0] == 8).all() and (C[1] == math.inf).all() and np.isnan(C[2]).all()
