"""Pins of the oracle's per-K-block scaled product (CPU only).

The tutorial's gemm_blockscaled applies SFA[M, ceil(K/g)] and SFB[N, ceil(K/g)]
along K one block of g at a time into a float32 accumulator.  Read for the
integer operands: the exact integer partial sum C_j of each block, term_j =
((float)C_j * SFA[m][j]) * SFB[n][j], added in increasing j into a binary32
accumulator (starting from term_0), every step rounding to nearest even, then
out().  Pinned here by: the one-block special case (the per-channel scaled
product, pinned on its own), unit scales (the exact integer GEMM), exact
rational brute force where no step rounds, hand-worked binary32 roundings
that fix the block order and the order of the two multiplies, the block of
each k (one-hot operands, distinct power-of-two scales per block, ragged
K), and row / column invariants of the two scale tables.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from precision_integer_gemm_amd.inputs import random_bytes

FMTS = [oracle.FMT_F32, oracle.FMT_BF16, oracle.FMT_F16]


def logical(stream, rows, K, lo=-8, hi=7):
    v = random_bytes(stream, rows * K).astype(np.int64) % (hi - lo + 1) + lo
    return v.astype(np.int8).reshape(rows, K)


def operands(variant, a_log, b_log):
    A = oracle.pack_int4(a_log) if variant == "i4i4" else a_log.copy()
    return A, oracle.pack_int4(b_log)


def nblocks(K, g):
    return -(-K // g)


@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
@pytest.mark.parametrize("fmt", FMTS)
def test_one_block_is_the_per_channel_product(variant, fmt):
    M, N, K = 7, 9, 96
    lo, hi = (-8, 7) if variant == "i4i4" else (-128, 127)
    a, b = logical(1, M, K, lo, hi), logical(2, N, K)
    A, B = operands(variant, a, b)
    rng = np.random.default_rng(3)
    sa = (rng.standard_normal(M) * 0.01).astype(np.float32)
    sb = (rng.standard_normal(N) * 3).astype(np.float32)
    want = oracle.gemm_scaled(variant, A, B, sa, sb, M, N, K, fmt)
    for g in (K, 128, 4096):                          # every g >= K is one block
        got = oracle.gemm_blockscaled(variant, A, B, sa.reshape(M, 1), sb.reshape(N, 1), M, N, K, g, fmt)
        assert np.array_equal(got, want)
        assert np.array_equal(np.signbit(got), np.signbit(want))


@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
@pytest.mark.parametrize("g", [32, 64, 128])
def test_unit_scales_give_the_integer_product(variant, g):
    # every partial sum is an integer below 2^24: no step rounds
    M, N, K = 5, 6, 320
    lo, hi = (-8, 7) if variant == "i4i4" else (-128, 127)
    a, b = logical(4, M, K, lo, hi), logical(5, N, K)
    A, B = operands(variant, a, b)
    nb = nblocks(K, g)
    got = oracle.gemm_blockscaled(variant, A, B, np.ones((M, nb), np.float32), np.ones((N, nb), np.float32),
                                  M, N, K, g, oracle.FMT_F32)
    exact = a.astype(np.int64) @ b.astype(np.int64).T             # the definition, by numpy
    assert np.array_equal(got, exact.astype(np.float64))


@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
def test_power_of_two_scales_match_exact_rationals(variant):
    # scales 2^e with e in [-3, 3]: every product is exact and every partial
    # sum stays below 2^24 in units of 2^-6, so the result is the exact
    # rational sum; computed here with Fractions from the logical values
    M, N, K, g = 4, 3, 200, 32
    lo, hi = (-8, 7) if variant == "i4i4" else (-64, 63)
    a, b = logical(6, M, K, lo, hi), logical(7, N, K)
    A, B = operands(variant, a, b)
    nb = nblocks(K, g)
    rng = np.random.default_rng(8)
    ea, eb = rng.integers(-3, 4, (M, nb)), rng.integers(-3, 4, (N, nb))
    sfa, sfb = np.ldexp(1.0, ea).astype(np.float32), np.ldexp(1.0, eb).astype(np.float32)
    got = oracle.gemm_blockscaled(variant, A, B, sfa, sfb, M, N, K, g, oracle.FMT_F32)
    for m in range(M):
        for n in range(N):
            s = Fraction(0)
            for k in range(K):
                j = k // g
                s += Fraction(int(a[m, k]) * int(b[n, k])) * Fraction(2) ** int(ea[m, j] + eb[n, j])
            assert Fraction(got[m, n]) == s


def rows_for_partials(partials, g):
    """Logical int4 rows (a, b) of len(partials) blocks whose block j sums to
    partials[j] >= 0: products (-8)*(-8) = 64, then 1*1."""
    K = g * len(partials)
    a = np.zeros((1, K), np.int8); b = np.zeros((1, K), np.int8)
    for j, p in enumerate(partials):
        q, r = divmod(p, 64)
        assert p >= 0 and q + r <= g
        for i in range(q + r):
            a[0, j * g + i] = b[0, j * g + i] = -8 if i < q else 1
    return a, b


def test_blocks_are_added_in_increasing_order():
    # partials 1, 2048, 1 with SFA = 1, 2^13, 1: terms 1, 2^24, 1.  In block
    # order, 1 + 2^24 is a tie between 2^24 and 2^24 + 2 and goes to the even
    # 2^24; adding 1 again ties again: the result is 2^24.  Any other order
    # that adds the two 1s first gives 2^24 + 2, and the exact sum is 2^24 + 2.
    g = 64
    a, b = rows_for_partials([1, 2048, 1], g)
    A, B = operands("i4i4", a, b)
    sfa = np.array([[1.0, 2.0 ** 13, 1.0]], np.float32)
    got = oracle.gemm_blockscaled("i4i4", A, B, sfa, np.ones((1, 3), np.float32), 1, 1, 3 * g, g,
                                  oracle.FMT_F32)
    assert got[0, 0] == 2.0 ** 24
    # reversed roles: the large term last; 1 + 1 = 2 exactly, 2 + 2^24 exact
    a, b = rows_for_partials([1, 1, 2048], g)
    A, B = operands("i4i4", a, b)
    sfa = np.array([[1.0, 1.0, 2.0 ** 13]], np.float32)
    got = oracle.gemm_blockscaled("i4i4", A, B, sfa, np.ones((1, 3), np.float32), 1, 1, 3 * g, g,
                                  oracle.FMT_F32)
    assert got[0, 0] == 2.0 ** 24 + 2


def test_multiply_order_within_a_block():
    # C_0 = 3, SFA = SFB = 1 + 2^-23.  (3 * SFA) = 3 + 1.5 ulp(3) (ulp 2^-22)
    # ties to the even 3 + 2^-21; times SFB: 3 + 3.5 ulp + 2^-44 rounds to
    # 3 + 2^-20.  Multiplying the scales first would give (1 + 2^-22) * 3 =
    # 3 + 3 * 2^-22.
    a, b = rows_for_partials([3], 32)
    A, B = operands("i4i4", a, b)
    s = np.array([[1.0 + 2.0 ** -23]], np.float32)
    got = oracle.gemm_blockscaled("i4i4", A, B, s, s, 1, 1, 32, 32, oracle.FMT_F32)
    assert got[0, 0] == 3.0 + 2.0 ** -20


@pytest.mark.parametrize("g", [32, 64, 128])
def test_each_k_uses_the_scale_of_its_block(g):
    # a single product a(0,k) b(n,k) = 1 per output column n = k; SFA[0][j] =
    # 2^j: D[0][k] = 2^(k // g), over a ragged K (last block partial)
    K = 5 * g + 34
    nb = nblocks(K, g)
    a = np.ones((1, K), np.int8)
    b = np.eye(K, dtype=np.int8)
    A, B = operands("i4i4", a, b)
    sfa = np.ldexp(1.0, np.arange(nb)).astype(np.float32).reshape(1, nb)
    got = oracle.gemm_blockscaled("i4i4", A, B, sfa, np.ones((K, nb), np.float32), 1, K, K, g,
                                  oracle.FMT_F32)
    assert np.array_equal(got[0], np.ldexp(1.0, np.arange(K) // g))
    # and SFB picks by the block of k as well: SFB[n][j] = 2^-j
    sfb = np.ldexp(1.0, -np.arange(nb)).astype(np.float32)[None, :].repeat(K, 0)
    got = oracle.gemm_blockscaled("i4i4", A, B, np.ones((1, nb), np.float32), sfb, 1, K, K, g,
                                  oracle.FMT_F32)
    assert np.array_equal(got[0], np.ldexp(1.0, -(np.arange(K) // g)))


@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
def test_scale_rows_act_on_rows_and_columns(variant):
    # doubling SFA row m doubles D row m; doubling SFB row n doubles D column
    # n (powers of two: exact, far from overflow); the scale tables' rows are
    # the output's rows and columns, not the other way round
    M, N, K, g = 6, 5, 192, 64
    lo, hi = (-8, 7) if variant == "i4i4" else (-128, 127)
    a, b = logical(9, M, K, lo, hi), logical(10, N, K)
    A, B = operands(variant, a, b)
    nb = nblocks(K, g)
    rng = np.random.default_rng(11)
    sfa = rng.uniform(0.5, 2, (M, nb)).astype(np.float32)
    sfb = rng.uniform(-2, 2, (N, nb)).astype(np.float32)
    base = oracle.gemm_blockscaled(variant, A, B, sfa, sfb, M, N, K, g, oracle.FMT_F32)
    sfa2 = sfa.copy(); sfa2[2] *= 2
    got = oracle.gemm_blockscaled(variant, A, B, sfa2, sfb, M, N, K, g, oracle.FMT_F32)
    want = base.copy(); want[2] *= 2
    assert np.array_equal(got, want)
    sfb2 = sfb.copy(); sfb2[4] *= 2
    got = oracle.gemm_blockscaled(variant, A, B, sfa, sfb2, M, N, K, g, oracle.FMT_F32)
    want = base.copy(); want[:, 4] *= 2
    assert np.array_equal(got, want)


def test_output_formats_round_the_binary32_result():
    # bf16 / f16 of the accumulated binary32 value: 1 + 2^-8 + 2^-10 (three
    # blocks, exact) rounds to 1 + 2^-7 in bf16 (above the tie) and stays in
    # f16 (11 bits); 70000 overflows f16 to infinity
    g = 32
    a, b = rows_for_partials([1, 1, 1], g)
    A, B = operands("i4i4", a, b)
    sfa = np.array([[1.0, 2.0 ** -8, 2.0 ** -10]], np.float32)
    one = np.ones((1, 3), np.float32)
    v = 1 + 2.0 ** -8 + 2.0 ** -10
    assert oracle.gemm_blockscaled("i4i4", A, B, sfa, one, 1, 1, 3 * g, g, oracle.FMT_BF16)[0, 0] == 1 + 2.0 ** -7
    assert oracle.gemm_blockscaled("i4i4", A, B, sfa, one, 1, 1, 3 * g, g, oracle.FMT_F16)[0, 0] == v
    sfa = np.array([[70000.0, 0.0, 0.0]], np.float32)
    assert oracle.gemm_blockscaled("i4i4", A, B, sfa, one, 1, 1, 3 * g, g, oracle.FMT_F16)[0, 0] == np.inf


def test_k_zero_and_argument_errors():
    out = oracle.gemm_blockscaled("i4i4", np.zeros((3, 0), np.uint8), np.zeros((2, 0), np.uint8),
                                  np.zeros((3, 0), np.float32), np.zeros((2, 0), np.float32), 3, 2, 0, 32,
                                  oracle.FMT_F32)
    assert (out == 0).all() and not np.signbit(out).any()
    with pytest.raises(ValueError):
        oracle.gemm_blockscaled("i4i4", np.zeros((1, 16), np.uint8), np.zeros((1, 16), np.uint8),
                                np.ones((1, 2), np.float32), np.ones((1, 1), np.float32), 1, 1, 32, 16,
                                oracle.FMT_F32)                   # SFB has the wrong width
    with pytest.raises(ValueError):
        oracle.gemm_blockscaled("i4i4", np.zeros((1, 16), np.uint8), np.zeros((1, 16), np.uint8),
                                np.ones((1, 1), np.float32), np.ones((1, 1), np.float32), 1, 1, 32, 0,
                                oracle.FMT_F32)
