"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each test fixes part of the oracle against what the pages or mathematics fix:
hand-worked fixtures under tests/golden/, an independent unpack formula, brute
force over every byte pair, closed forms, invariants and numpy's int64 matmul.
A plausible slip anywhere in the oracle (nibble order swapped, sign extension
dropped, an operand transposed, a term dropped, int32 overflow) fails at least
one of them.
"""
import os

import numpy as np
import pytest

import oracle
from precision_integer_gemm_amd.inputs import custom_operands, random_bytes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


# -- independent numpy unpack: the shift-pair sign extension of the w4a8 page
#    (field moved to the top of an int8, then an arithmetic right shift), a
#    different formula from the oracle's subtract-16.
def np_unpack(packed):
    b = np.ascontiguousarray(packed).view(np.uint8)
    lo = ((b << 4).astype(np.uint8)).view(np.int8) >> 4
    hi = b.view(np.int8) >> 4
    return np.stack([lo, hi], axis=-1).reshape(b.shape[0], -1)


def np_gemm(a, b):
    return a.astype(np.int64) @ b.astype(np.int64).T


# P1 -- all 16 nibble values ---------------------------------------------------
def test_nibble_table_all_16_values():
    table = {int(bits, 2): int(v) for bits, v in _lines("int4_nibble_table.txt")}
    assert sorted(table) == list(range(16))
    # low nibble: byte = field; high nibble: byte = field << 4
    lo_bytes = np.array([[f for f in range(16)]], dtype=np.uint8)
    hi_bytes = np.array([[f << 4 for f in range(16)]], dtype=np.uint8)
    lo = oracle.unpack_int4(lo_bytes, 32)[0, 0::2]
    hi = oracle.unpack_int4(hi_bytes, 32)[0, 1::2]
    assert lo.tolist() == [table[f] for f in range(16)]
    assert hi.tolist() == [table[f] for f in range(16)]
    # the zero nibble of each byte decodes to 0
    assert not oracle.unpack_int4(lo_bytes, 32)[0, 1::2].any()
    assert not oracle.unpack_int4(hi_bytes, 32)[0, 0::2].any()


def test_unpack_matches_shift_pair_formula_on_all_bytes():
    allb = np.arange(256, dtype=np.uint8).reshape(1, 256)
    assert np.array_equal(oracle.unpack_int4(allb, 512), np_unpack(allb))


# P2 / P8 -- pack: hand-worked bytes, round trip, bijection, page's shape ------
def test_pack_worked_examples():
    for row in _lines("pack_worked.txt"):
        if row[0] == "shape":
            continue
        even, odd, hexbyte = int(row[0]), int(row[1]), int(row[2], 16)
        packed = oracle.pack_int4(np.array([[even, odd]], dtype=np.int8))
        assert packed.tolist() == [[hexbyte]], row
        assert oracle.unpack_int4(packed, 2).tolist() == [[even, odd]], row


def test_pack_shape_printed_by_tutorial():
    rows = [r for r in _lines("pack_worked.txt") if r[0] == "shape"]
    assert rows == [["shape", "1024", "1024", "->", "1024", "512"]]
    logical = (random_bytes(7, 1024 * 1024).view(np.int8) >> 4).reshape(1024, 1024)
    assert oracle.pack_int4(logical).shape == (1024, 512)


def test_pack_unpack_round_trip_all_pairs_and_bytes():
    vals = np.arange(-8, 8, dtype=np.int8)
    ev, od = np.meshgrid(vals, vals, indexing="ij")
    logical = np.stack([ev.ravel(), od.ravel()], axis=-1).reshape(1, 512)
    packed = oracle.pack_int4(logical)
    assert packed.shape == (1, 256)
    assert sorted(packed.ravel().tolist()) == list(range(256))  # bijection
    assert np.array_equal(oracle.unpack_int4(packed, 512), logical)
    allb = np.arange(256, dtype=np.uint8).reshape(1, 256)
    assert np.array_equal(oracle.pack_int4(oracle.unpack_int4(allb, 512)), allb)


def test_pack_argument_errors_like_the_page():
    with pytest.raises(TypeError):
        oracle.pack_int4(np.zeros((2, 4), dtype=np.int16))
    with pytest.raises(ValueError):
        oracle.pack_int4(np.zeros((2, 3), dtype=np.int8))
    with pytest.raises(ValueError):
        oracle.pack_int4(np.int8(1))


# hand-worked products --------------------------------------------------------
def _worked_cases():
    cases, cur = [], None
    for row in _lines("gemm_worked.txt"):
        if row[0] == "case":
            cur = {"variant": row[1], "M": int(row[2]), "N": int(row[3]), "K": int(row[4]),
                   "A": [], "B": [], "C": []}
            cases.append(cur)
        elif row[0] in ("A", "B"):
            cur[row[0]].append([int(x, 16) for x in row[1:]])
        elif row[0] == "C":
            cur["C"].append([int(x) for x in row[1:]])
    return cases


@pytest.mark.parametrize("case", _worked_cases(), ids=lambda c: c["variant"])
def test_hand_worked_products(case):
    A = np.array(case["A"], dtype=np.uint8)
    B = np.array(case["B"], dtype=np.uint8)
    M, N, K = case["M"], case["N"], case["K"]
    if case["variant"] == "i4i4":
        C = oracle.gemm_i4i4(A, B, M, N, K)
    else:
        C = oracle.gemm_w4a8(A.view(np.int8), B, M, N, K)
    assert C.tolist() == case["C"]
    ms, ns = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    fn = oracle.gemm_i4i4_at if case["variant"] == "i4i4" else oracle.gemm_w4a8_at
    arg_a = A if case["variant"] == "i4i4" else A.view(np.int8)
    assert fn(arg_a, B, M, N, K, ms.ravel(), ns.ravel()).reshape(M, N).tolist() == case["C"]


# P3 -- brute force over every byte pair at K = 2 -------------------------------
def test_brute_force_i4i4_all_byte_pairs_k2():
    allb = np.arange(256, dtype=np.uint8).reshape(256, 1)
    C = oracle.gemm_i4i4(allb, allb, 256, 256, 2)
    v = np_unpack(allb)  # [256, 2]: (lo, hi) of each byte
    want = np.outer(v[:, 0], v[:, 0]).astype(np.int64) + np.outer(v[:, 1], v[:, 1])
    assert np.array_equal(C, want)


def test_brute_force_w4a8_all_pairs_k2():
    # every (a0, a1) int8 pair against every B byte: 65536 x 256 products
    a = np.stack(np.meshgrid(np.arange(-128, 128), np.arange(-128, 128), indexing="ij"),
                 axis=-1).reshape(65536, 2).astype(np.int8)
    allb = np.arange(256, dtype=np.uint8).reshape(256, 1)
    C = oracle.gemm_w4a8(a, allb, 65536, 256, 2)
    v = np_unpack(allb).astype(np.int64)
    want = np.outer(a[:, 0], v[:, 0]) + np.outer(a[:, 1].astype(np.int64), v[:, 1])
    assert np.array_equal(C, want)


# P4 -- independent numpy int64 matmul on small and ragged shapes ---------------
SHAPES = [(1, 1, 2), (3, 5, 2), (7, 9, 30), (17, 33, 34), (37, 53, 86), (64, 64, 64),
          (16, 48, 128), (5, 3, 258)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_i4i4_matches_numpy(M, N, K):
    A, B = custom_operands("i4i4", M, N, K, seed=100 + M)
    want = np_gemm(np_unpack(A), np_unpack(B))
    assert np.array_equal(oracle.gemm_i4i4(A, B, M, N, K), want)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_w4a8_matches_numpy(M, N, K):
    A, B = custom_operands("w4a8", M, N, K, seed=200 + M)
    want = np_gemm(A, np_unpack(B))
    assert np.array_equal(oracle.gemm_w4a8(A, B, M, N, K), want)


@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
def test_sampled_elements_match_full_product(variant):
    M, N, K = 45, 71, 198
    A, B = custom_operands(variant, M, N, K, seed=9)
    full = (oracle.gemm_i4i4 if variant == "i4i4" else oracle.gemm_w4a8)(A, B, M, N, K)
    rng = np.random.default_rng(0)
    ms, ns = rng.integers(0, M, 500), rng.integers(0, N, 500)
    at = (oracle.gemm_i4i4_at if variant == "i4i4" else oracle.gemm_w4a8_at)
    assert np.array_equal(at(A, B, M, N, K, ms, ns), full[ms, ns])


# P5 -- closed forms -----------------------------------------------------------
def _packed_const(rows, K, v):
    nib = v & 0xF
    return np.full((rows, K // 2), nib | (nib << 4), dtype=np.uint8)


@pytest.mark.parametrize("K", [2, 64, 1000, 8192])
def test_closed_forms_constant_operands(K):
    M, N = 3, 4
    m8 = _packed_const(M, K, -8)
    assert (oracle.gemm_i4i4(m8, _packed_const(N, K, -8), M, N, K) == 64 * K).all()
    assert (oracle.gemm_i4i4(m8, _packed_const(N, K, 7), M, N, K) == -56 * K).all()
    assert (oracle.gemm_i4i4(_packed_const(M, K, 1), _packed_const(N, K, 1), M, N, K) == K).all()
    a_min = np.full((M, K), -128, dtype=np.int8)
    a_max = np.full((M, K), 127, dtype=np.int8)
    assert (oracle.gemm_w4a8(a_min, _packed_const(N, K, -8), M, N, K) == 1024 * K).all()
    assert (oracle.gemm_w4a8(a_max, _packed_const(N, K, 7), M, N, K) == 889 * K).all()
    assert (oracle.gemm_w4a8(a_min, _packed_const(N, K, 7), M, N, K) == -896 * K).all()
    assert (oracle.gemm_w4a8(np.ones((M, K), np.int8), _packed_const(N, K, 1), M, N, K) == K).all()


@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
@pytest.mark.parametrize("K", [64, 256, 2080])
def test_one_odd_term_closed_form(variant, K):
    # extreme operands with a single 1 per row: 64 K - 144, or the odd 64 K - 63
    # where the two positions meet (1024 K - 2184 / 1024 K - 1023 for W4A8);
    # the GPU tests use the same family at the largest K
    from closed_forms import odd_term_operands, odd_term_product
    M, N = 13, 29
    A, B, p, q = odd_term_operands(variant, M, N, K)
    want = odd_term_product(variant, K, p, q)
    assert (want[p[:, None] == q[None, :]] % 2 == 1).all() and (p[:, None] == q[None, :]).any()
    fn = oracle.gemm_i4i4 if variant == "i4i4" else oracle.gemm_w4a8
    assert np.array_equal(fn(A, B, M, N, K), want)
    a_logical = np_unpack(A) if variant == "i4i4" else A
    assert np.array_equal(np_gemm(a_logical, np_unpack(B)), want)


def _identity_like_packed(N, K):
    # B[n][k] = 1 if n == k else 0
    logical = np.zeros((N, K), dtype=np.int8)
    for n in range(min(N, K)):
        logical[n, n] = 1
    return oracle.pack_int4(logical)


@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
def test_identity_like_b_returns_columns_of_a(variant):
    M, N, K = 9, 40, 34  # N > K: columns past K are zero
    A, _ = custom_operands(variant, M, N, K, seed=11)
    B = _identity_like_packed(N, K)
    a_logical = np_unpack(A) if variant == "i4i4" else A
    fn = oracle.gemm_i4i4 if variant == "i4i4" else oracle.gemm_w4a8
    C = fn(A, B, M, N, K)
    assert np.array_equal(C[:, :K], a_logical.astype(np.int32))
    assert not C[:, K:].any()


def test_permutation_b_permutes_columns():
    M, N, K = 6, 20, 20
    A, _ = custom_operands("w4a8", M, N, K, seed=12)
    perm = np.random.default_rng(1).permutation(K)
    logical = np.zeros((N, K), dtype=np.int8)
    logical[np.arange(N), perm] = 1
    C = oracle.gemm_w4a8(A, oracle.pack_int4(logical), M, N, K)
    assert np.array_equal(C, A[:, perm].astype(np.int32))


def test_rank_one_and_alternating_sign():
    M, N, K = 5, 6, 48
    u = np.array([-8, -3, 0, 4, 7], dtype=np.int8)
    v = np.array([7, -8, 1, 2, -1, 5], dtype=np.int8)
    A = oracle.pack_int4(np.repeat(u[:, None], K, axis=1))
    B = oracle.pack_int4(np.repeat(v[:, None], K, axis=1))
    assert np.array_equal(oracle.gemm_i4i4(A, B, M, N, K), K * np.outer(u, v).astype(np.int32))
    alt = np.tile(np.array([1, -1], dtype=np.int8), (N, K // 2))  # b = (-1)^k
    C = oracle.gemm_w4a8(np.ones((M, K), np.int8), oracle.pack_int4(alt), M, N, K)
    assert not C.any()
    # only odd k survives when a = (k odd): sum of b over odd k = -K/2
    a_odd = np.tile(np.array([0, 1], dtype=np.int8), (M, K // 2))
    assert (oracle.gemm_w4a8(a_odd, oracle.pack_int4(alt), M, N, K) == -K // 2).all()


# P6 -- invariants ---------------------------------------------------------------
def test_transpose_symmetry_i4i4():
    M, N, K = 23, 31, 66
    A, B = custom_operands("i4i4", M, N, K, seed=13)
    assert np.array_equal(oracle.gemm_i4i4(A, B, M, N, K), oracle.gemm_i4i4(B, A, N, M, K).T)


def test_w4a8_equals_i4i4_when_a_fits_int4():
    M, N, K = 19, 27, 62
    _, B = custom_operands("i4i4", M, N, K, seed=14)
    a8 = (random_bytes(99, M * K).view(np.int8) >> 4).reshape(M, K)  # values in [-8, 7]
    assert np.array_equal(oracle.gemm_w4a8(a8, B, M, N, K),
                          oracle.gemm_i4i4(oracle.pack_int4(a8), B, M, N, K))


@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
def test_k_additivity(variant):
    M, N, K, K1 = 11, 13, 96, 34
    A, B = custom_operands(variant, M, N, K, seed=15)
    fn = oracle.gemm_i4i4 if variant == "i4i4" else oracle.gemm_w4a8
    acols = K // 2 if variant == "i4i4" else K
    a1 = A[:, : (K1 // 2 if variant == "i4i4" else K1)]
    a2 = A[:, (K1 // 2 if variant == "i4i4" else K1):acols]
    full = fn(A, B, M, N, K).astype(np.int64)
    part = fn(a1, B[:, : K1 // 2], M, N, K1).astype(np.int64) + \
        fn(a2, B[:, K1 // 2:], M, N, K - K1)
    assert np.array_equal(full, part)


def test_row_prefix_case_reuses_rows():
    K, N = 256, 40
    A16, B = custom_operands("w4a8", 16, N, K, seed=4)
    A1, B1 = custom_operands("w4a8", 1, N, K, seed=4)
    assert np.array_equal(A1, A16[:1]) and np.array_equal(B1, B)
    assert np.array_equal(oracle.gemm_w4a8(A1, B, 1, N, K), oracle.gemm_w4a8(A16, B, 16, N, K)[:1])


# P7 -- overflow envelope and degenerate shapes ----------------------------------
def test_envelope_and_range_check():
    M, N, K = 8, 8, 4096
    A, B = custom_operands("w4a8", M, N, K, seed=16)
    assert np.abs(oracle.gemm_w4a8(A, B, M, N, K)).max() <= 1024 * K
    A, B = custom_operands("i4i4", M, N, K, seed=16)
    assert np.abs(oracle.gemm_i4i4(A, B, M, N, K)).max() <= 64 * K
    # a sum outside int32 is reported, not wrapped: 1024 * K > 2^31 - 1
    K = 2 ** 21 + 2
    a = np.full((1, K), -128, dtype=np.int8)
    with pytest.raises(ValueError, match="int32"):
        oracle.gemm_w4a8(a, _packed_const(1, K, -8), 1, 1, K)


def test_degenerate_shapes():
    assert oracle.gemm_i4i4(np.zeros((0, 2), np.uint8), np.zeros((3, 2), np.uint8), 0, 3, 4).shape == (0, 3)
    C = oracle.gemm_w4a8(np.zeros((2, 0), np.int8), np.zeros((3, 0), np.uint8), 2, 3, 0)
    assert C.shape == (2, 3) and not C.any()
    with pytest.raises(ValueError):
        oracle.gemm_i4i4(np.zeros((1, 2), np.uint8), np.zeros((1, 2), np.uint8), 1, 1, 3)
