"""Pins of the oracle's fp8 (e4m3) GEMM: decode, encode and the product.

The e4m3 decode is checked against PyTorch's float8_e4m3fn (an independent
implementation of the same OCP format) and against values the format's
definition fixes; the encode against PyTorch's nearest-even conversion inside
the finite range and against the saturating reading above it; the product
against exact rational arithmetic on small shapes and closed forms.
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
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_encode(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_torch_on_every_code():
    got, want = oracle.fp8_e4m3_decode(ALL), torch_decode(ALL)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


@pytest.mark.parametrize("code,value", [
    (0x38, 1.0), (0x40, 2.0), (0x3F, 1.875), (0x7E, 448.0), (0xFE, -448.0),
    (0x08, 2.0 ** -6), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x00, 0.0),
])
def test_decode_definition_values(code, value):
    assert oracle.fp8_e4m3_decode(np.array([code], np.uint8))[0] == value


def test_decode_nan_and_signed_zero():
    v = oracle.fp8_e4m3_decode(np.array([0x7F, 0xFF, 0x80], np.uint8))
    assert math.isnan(v[0]) and math.isnan(v[1])
    assert v[2] == 0.0 and math.copysign(1.0, v[2]) < 0


def test_encode_round_trips_every_finite_code():
    finite = ALL[~np.isnan(torch_decode(ALL))]
    assert np.array_equal(oracle.fp8_e4m3_encode(oracle.fp8_e4m3_decode(finite)), finite)


def test_encode_midpoints_and_random_values_match_torch():
    vals = np.sort(np.unique(torch_decode(ALL)[~np.isnan(torch_decode(ALL))]))
    mids = (vals[:-1] + vals[1:]) / 2                      # every tie, both signs
    rng = np.random.default_rng(8)
    rand = rng.uniform(-464.0, 464.0, 20000).astype(np.float32).astype(np.float64)
    tiny = rng.uniform(-2.0 ** -5, 2.0 ** -5, 5000).astype(np.float32).astype(np.float64)
    for x in (mids, rand, tiny, np.array([464.0, -464.0, 460.0])):
        assert np.array_equal(oracle.fp8_e4m3_encode(x), torch_encode(x))


def test_encode_saturates_beyond_the_finite_range():
    # the finite-saturating reading: every magnitude above 448 gives +-448
    x = np.array([448.5, 465.0, 480.0, 1e6, math.inf, -500.0, -math.inf])
    assert oracle.fp8_e4m3_encode(x).tolist() == [0x7E] * 5 + [0xFE] * 2
    assert oracle.fp8_e4m3_encode(np.array([math.nan]))[0] & 0x7F == 0x7F


def finite_codes(stream, n):
    c = random_bytes(stream, n)
    return np.where((c & 0x7F) == 0x7F, c & 0xF8, c).astype(np.uint8)  # replace NaN codes


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (2, 3, 5), (4, 3, 16), (3, 5, 33)])
def test_gemm_matches_exact_rational_brute_force(M, N, K):
    A = finite_codes(100 + M, M * K).reshape(M, K)
    B = finite_codes(200 + N, N * K).reshape(N, K)
    C, Cabs = oracle.gemm_fp8(A, B, M, N, K)
    da = [[Fraction(v) for v in row] for row in torch_decode(A)]
    db = [[Fraction(v) for v in row] for row in torch_decode(B)]
    for m in range(M):
        for n in range(N):
            s = sum(da[m][k] * db[n][k] for k in range(K))
            sa = sum(abs(da[m][k] * db[n][k]) for k in range(K))
            assert Fraction(C[m, n]) == s and Fraction(Cabs[m, n]) == sa


def test_gemm_closed_forms():
    K = 4096
    ones = np.full((3, K), 0x38, np.uint8)                       # 1.0
    C, Cabs = oracle.gemm_fp8(ones, ones[:2], 3, 2, K)
    assert (C == K).all() and (Cabs == K).all()
    big, nbig = np.full((2, K), 0x7E, np.uint8), np.full((2, K), 0xFE, np.uint8)
    C, Cabs = oracle.gemm_fp8(big, nbig, 2, 2, K)               # 448 * -448 each
    assert (C == -200704.0 * K).all() and (Cabs == 200704.0 * K).all()
    # one-hot rows of B pick columns of A
    M, N, K = 5, 4, 64
    A = finite_codes(7, M * K).reshape(M, K)
    B = np.zeros((N, K), np.uint8)
    cols = [0, 7, 31, 63]
    for n, j in enumerate(cols):
        B[n, j] = 0x38
    C, _ = oracle.gemm_fp8(A, B, M, N, K)
    assert np.array_equal(C, torch_decode(A)[:, cols])


def test_gemm_nan_operand_gives_nan():
    A = np.full((2, 8), 0x38, np.uint8)
    A[1, 3] = 0x7F
    C, _ = oracle.gemm_fp8(A, np.full((2, 8), 0x38, np.uint8), 2, 2, 8)
    assert not np.isnan(C[0]).any() and np.isnan(C[1]).all()


def test_group_exponent_bound_helper():
    # the matrix-core error bound used by the GPU tests, against a hand-worked
    # value and a per-group brute force over the products' exponent sums
    import sys, os
    sys.path.insert(0, os.path.dirname(__file__))
    from fp8_bounds import group_exponent_bound
    a = np.zeros((1, 16)); b = np.zeros((1, 16))
    a[0, 0], a[0, 3], b[0, 1], b[0, 9] = 448.0, 1.0, 448.0, 2.0 ** -9   # group 1 of A is empty
    A, B = oracle.fp8_e4m3_encode(a).reshape(1, 16), oracle.fp8_e4m3_encode(b).reshape(1, 16)
    assert group_exponent_bound(A, B, 16)[0, 0] == 7 * 2.0 ** (8 + 8 - 13)
    rng = np.random.default_rng(3)
    M, N, K = 5, 6, 40
    A = rng.integers(0, 256, (M, K)).astype(np.uint8); B = rng.integers(0, 256, (N, K)).astype(np.uint8)
    A[(A & 0x7F) == 0x7F] &= 0xF8; B[(B & 0x7F) == 0x7F] &= 0xF8
    A[:, 8:16] = 0                                                     # an empty group
    ex = lambda c: np.where(((c >> 3) & 15) == 0, -6, ((c >> 3) & 15).astype(int) - 7)
    got = group_exponent_bound(A, B, K)
    for m in range(M):
        for n in range(N):
            exact = 0.0   # with the per-product exponent sum E of each group
            for g in range(K // 8):
                ks = [k for k in range(8 * g, 8 * g + 8) if (A[m, k] & 0x7F) and (B[n, k] & 0x7F)]
                if ks:
                    exact += 7 * 2.0 ** (max(int(ex(A[m, k])) + int(ex(B[n, k])) for k in ks) - 13)
            assert got[m, n] >= exact
            assert got[m, n] <= 2.0 ** 14 * max(exact, 2.0 ** -30)
