"""Seeded synthetic inputs for the low-precision GEMM workloads.

This module only draws random bytes; it holds none of the GEMM's arithmetic
(no packing, unpacking or products).  Both the GPU path and the CPU oracle are
fed the bytes it returns.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), used counter-style: output i of stream s is
mix(s + (i + 1) * 0x9E3779B97F4A7C15) with the published mix function.  Each
64-bit output gives 8 bytes, least significant first.

Value distributions follow the pages' workloads:
  * an int8 operand is uniform over [-128, 127]: one random byte per element;
  * a packed int4 operand holds logical values uniform over [-8, 7] (the
    tutorial draws randint(-8, 8)); since every 4-bit pattern is one of the 16
    values, independent uniform nibbles are exactly uniform random bytes, so
    the packed bytes are drawn directly, both nibbles of every byte populated.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(stream: int, count: int, start: int = 0) -> np.ndarray:
    """Outputs start .. start+count-1 of SplitMix64 seeded with `stream`."""
    with np.errstate(over="ignore"):
        i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = np.uint64(stream & 0xFFFFFFFFFFFFFFFF) + i * _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def random_bytes(stream: int, nbytes: int) -> np.ndarray:
    """`nbytes` uniform random bytes (uint8) from SplitMix64 stream `stream`."""
    words = splitmix64(stream, (nbytes + 7) // 8)
    return words.astype("<u8").view(np.uint8)[:nbytes].copy()


def operand_stream(seed: int, operand: int) -> int:
    """Stream id of operand 0 (A) or 1 (B) of the case seeded `seed`."""
    return (seed << 8) | operand


@dataclass(frozen=True)
class Case:
    name: str
    variant: str  # "i4i4" or "w4a8"
    M: int
    N: int
    K: int
    seed: int
    a_rows_from: str | None = None  # reuse another case's A rows (prefix)

    @property
    def ops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def a_bytes(self) -> int:
        return self.M * (self.K // 2 if self.variant == "i4i4" else self.K)

    @property
    def b_bytes(self) -> int:
        return self.N * self.K // 2

    @property
    def c_bytes(self) -> int:
        return 4 * self.M * self.N

    @property
    def alg_bytes(self) -> int:
        return self.a_bytes + self.b_bytes + self.c_bytes


# The workloads: shapes and value distributions of the pages' examples (the
# int4 example's default 1024^3, square compute-bound shapes, a decode-like
# skinny W4A8 shape and a ragged one).  Seeds are the case numbers.
CASES = {
    "i4i4_256": Case("i4i4_256", "i4i4", 256, 256, 256, 1),
    "i4i4_1024": Case("i4i4_1024", "i4i4", 1024, 1024, 1024, 2),
    "w4a8_4096": Case("w4a8_4096", "w4a8", 4096, 4096, 4096, 3),
    "w4a8_skinny_m16": Case("w4a8_skinny_m16", "w4a8", 16, 28672, 8192, 4),
    "w4a8_skinny_m1": Case("w4a8_skinny_m1", "w4a8", 1, 28672, 8192, 4,
                           a_rows_from="w4a8_skinny_m16"),
    "i4i4_8192": Case("i4i4_8192", "i4i4", 8192, 8192, 8192, 5),
    "i4i4_ragged": Case("i4i4_ragged", "i4i4", 3000, 5120, 6144, 6),
}


def operands(case: Case) -> tuple[np.ndarray, np.ndarray]:
    """Host bytes (A, B) of a case: A is int8 [M,K] (w4a8) or packed uint8
    [M,K/2] (i4i4); B is packed uint8 [N,K/2].  A case with `a_rows_from`
    takes the first M rows of that case's A and the same B (same seed)."""
    a_row_bytes = case.K // 2 if case.variant == "i4i4" else case.K
    a = random_bytes(operand_stream(case.seed, 0), case.M * a_row_bytes)
    a = a.reshape(case.M, a_row_bytes)
    if case.variant == "w4a8":
        a = a.view(np.int8)
    b = random_bytes(operand_stream(case.seed, 1), case.N * case.K // 2)
    return a, b.reshape(case.N, case.K // 2)


def custom_operands(variant: str, M: int, N: int, K: int, seed: int):
    """Operands of an ad-hoc shape (tests), drawn like the named cases."""
    return operands(Case("custom", variant, M, N, K, seed))


def scale_vector(seed: int, which: int, n: int, lo_exp: int = -12, hi_exp: int = 0) -> np.ndarray:
    """`n` float32 scales for the scaled product (which = 0: per row of A,
    1: per row of B): random sign, a random binary exponent in
    [lo_exp, hi_exp] and a random 23-bit mantissa, so the epilogue's
    roundings are exercised.  Drawn from stream (seed << 8) | (2 + which)."""
    words = splitmix64(operand_stream(seed, 2 + which), n)
    sign = (words >> np.uint64(63)).astype(np.uint32)
    span = hi_exp - lo_exp + 1
    exp = (words >> np.uint64(32)).astype(np.uint64) % np.uint64(span)
    biased = (exp.astype(np.int64) + lo_exp + 127).astype(np.uint32)
    mant = (words & np.uint64(0x7FFFFF)).astype(np.uint32)
    bits = (sign << np.uint32(31)) | (biased << np.uint32(23)) | mant
    return bits.view(np.float32)


def block_scale_table(seed: int, which: int, rows: int, K: int, g: int, lo_exp: int = -12,
                      hi_exp: int = 0) -> np.ndarray:
    """float32 scales [rows, ceil(K / g)] for the per-K-block scaled product
    (which = 0: SFA, 1: SFB), drawn like scale_vector (random sign, exponent in
    [lo_exp, hi_exp], random 23-bit mantissa) from the same streams."""
    nb = -(-K // g)
    return scale_vector(seed, which, rows * nb, lo_exp, hi_exp).reshape(rows, nb)


def fp8_codes(seed: int, which: int, rows: int, K: int, fmt: str = "e4m3") -> np.ndarray:
    """Uniform random fp8 bytes [rows, K] for the fp8 workload (which = 0: A,
    1: B), drawn from stream (seed << 8) | which, every operand finite: for
    e4m3 the two NaN codes (S.1111.111) are replaced by the code with the
    same sign and exponent and mantissa 0; for e5m2 the infinity and NaN codes
    (exponent field 31) by the codes of the largest finite binade with the
    same sign and mantissa."""
    c = random_bytes(operand_stream(seed, which), rows * K)
    if fmt == "e4m3":
        c = np.where((c & 0x7F) == 0x7F, c & 0xF8, c)
    elif fmt == "e5m2":
        c = np.where((c & 0x7C) == 0x7C, c & 0xFB, c)
    else:
        raise ValueError(f"unknown fp8 format {fmt!r}")
    return c.astype(np.uint8).reshape(rows, K)
