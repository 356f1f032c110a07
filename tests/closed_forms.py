"""Operands with a known product, shared by the CPU pins and the GPU tests.

One-odd-term family.  Every element of A and B is the most negative value of
its format (-8 for a 4-bit operand, -128 for an int8 A) except one position
per row: a(m, p[m]) = 1 and b(n, q[n]) = 1.  Then

    C[m][n] = K * x * y  - (x * y - x) - (x * y - y) + [p[m] == q[n]] * (x * y - x - y + 1)

with x the extreme value of A and y = -8 that of B: where the positions meet,
one term is 1 * 1 instead of x * y; where they do not, one term is 1 * y and
another x * 1.  For int4 x int4 (x = y = -8) that is 64 K - 144, or the odd
value 64 K - 63 where the positions meet.  At the largest K that the library
accepts, K = 131040 (a multiple of 32), the odd value is 8386497: the
accumulator holds 64 (K - 1) = 8386496 < 2^23 before or after the single
product 1, so a sum that dropped a low-order unit next to a large partial sum
would show.  This family is how the exactness of the fp32 accumulation on
the FP6 matrix cores is checked.
"""
import numpy as np


def odd_term_positions(K: int):
    """Positions inside the first, a middle and the last 64-k block, at both
    halves of a 32-k lane group and both nibbles of a byte."""
    cand = [0, 1, 31, 32, 63, K // 2, K // 2 + 33, K - 64, K - 33, K - 32, K - 2, K - 1]
    out = []
    for p in cand:
        if 0 <= p < K and p not in out:
            out.append(p)
    return out


def odd_term_operands(variant: str, M: int, N: int, K: int):
    """(A, B, p, q): A as packed bytes [M, K/2] (int4 x int4) or int8 [M, K]
    (W4A8), B packed [N, K/2], and the positions of the 1s."""
    pos = odd_term_positions(K)
    p = np.array([pos[m % len(pos)] for m in range(M)], dtype=np.int64)
    # a different stride for the columns, so every pair of positions occurs
    q = np.array([pos[(5 * n + n // len(pos)) % len(pos)] for n in range(N)], dtype=np.int64)

    def packed_with_ones(rows, where):
        X = np.full((rows, K // 2), 0x88, dtype=np.uint8)  # both nibbles -8
        for r, k in enumerate(where):
            X[r, k // 2] = 0x81 if k % 2 == 0 else 0x18    # the nibble of k becomes 1
        return X

    B = packed_with_ones(N, q)
    if variant == "i4i4":
        A = packed_with_ones(M, p)
    else:
        A = np.full((M, K), -128, dtype=np.int8)
        A[np.arange(M), p] = 1
    return A, B, p, q


def odd_term_product(variant: str, K: int, p, q) -> np.ndarray:
    """The closed form of the one-odd-term product, int64 [len(p), len(q)]."""
    x = -8 if variant == "i4i4" else -128
    y = -8
    meet = (np.asarray(p)[:, None] == np.asarray(q)[None, :]).astype(np.int64)
    base = K * x * y - (x * y - x) - (x * y - y)
    return base + meet * (x * y - x - y + 1)
