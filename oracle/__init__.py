"""CPU oracle for the low-precision integer GEMM C[M,N] = A[M,K] . B[N,K]^T.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``, the smoke check
in ``__graft_entry__`` and the benchmark's CPU-baseline leg may import this
module.  It shares no code with the GPU library; the two meet only through the
seeded input bytes that both are given.

The arithmetic lives in ``lpgemm_oracle.c`` (plain C, int64 accumulation, see
its header for the passages of the pages it follows).  This module builds it
with gcc and marshals numpy arrays through ctypes; it does no arithmetic of its
own.

Pages cited (by title):
  * tilelang PR "[CUDA] Support int4 T.gemm" (#2063), example gemm_int4.
  * tilelang PR "[Example] add w4a8 gemm kernel" (#815), reviews of
    torch_convert / ref_program.
  * TileLang tutorial ch. 14 sec. 5 "low_precision_gemm.py", pack_int4,
    matmul_int4, gemm_blockscaled (the scaled epilogue with one K block, and
    the per-K-block scaled product) and
    gemm_fp8 (the fp8 GEMM: e4m3 operands, fp32 accumulation, fp8 C).

Every function here is pinned: the integer GEMMs and pack/unpack by
``tests/test_oracle_pins.py`` (hand-worked values, closed forms, brute force,
an independent numpy computation), the scaled epilogue by
``tests/test_oracle_scaled.py``, the per-K-block product by
``tests/test_oracle_blockscaled.py``, the e4m3 decode/encode and the fp8 product by
``tests/test_oracle_fp8.py`` (PyTorch's float8_e4m3fn, exact rationals, closed
forms); ``tests/test_oracle_mutants.py`` checks that planted mistakes fail
them.  No function is left unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lpgemm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_lpgemm_oracle.so")

_ERRORS = {1: "invalid argument", 2: "result outside int32", 3: "out of host memory"}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP over the outer row loop)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_num_threads.restype = ctypes.c_int
    for name in ("oracle_fp8_e5m2_decode",):
        f = getattr(lib, name)
        f.argtypes = [p, i64, p]
        f.restype = ctypes.c_int
    lib.oracle_fp8_e5m2_encode.argtypes = [p, i64, p]
    lib.oracle_fp8_e5m2_encode.restype = ctypes.c_int
    lib.oracle_gemm_fp8_e5m2.argtypes = [p, p, i64, i64, i64, p, p]
    lib.oracle_gemm_fp8_e5m2.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
    for name in ("oracle_unpack_int4", "oracle_pack_int4"):
        f = getattr(lib, name)
        f.argtypes = [p, i64, i64, p]
        f.restype = ctypes.c_int
    for name in ("oracle_gemm_i4i4", "oracle_gemm_w4a8"):
        f = getattr(lib, name)
        f.argtypes = [p, p, i64, i64, i64, p]
        f.restype = ctypes.c_int
    lib.oracle_scaled_epilogue.argtypes = [p, p, p, i64, i64, ctypes.c_int, p]
    lib.oracle_scaled_epilogue.restype = ctypes.c_int
    for name in ("oracle_gemm_i4i4_at", "oracle_gemm_w4a8_at"):
        f = getattr(lib, name)
        f.argtypes = [p, p, i64, i64, i64, p, p, i64, p]
        f.restype = ctypes.c_int
    for name in ("oracle_fp8_e4m3_decode", "oracle_fp8_e4m3_encode"):
        f = getattr(lib, name)
        f.argtypes = [p, i64, p]
        f.restype = ctypes.c_int
    lib.oracle_gemm_fp8.argtypes = [p, p, i64, i64, i64, p, p]
    lib.oracle_gemm_blockscaled.argtypes = [ctypes.c_int, p, p, p, p, i64, i64, i64, i64, ctypes.c_int, p]
    lib.oracle_gemm_fp8.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what}: {_ERRORS.get(rc, rc)}")


def _bytes2d(x, rows: int, cols: int, name: str) -> np.ndarray:
    """View an (int8 or uint8) array as contiguous uint8 [rows, cols]."""
    a = np.ascontiguousarray(x)
    if a.dtype not in (np.int8, np.uint8):
        raise TypeError(f"{name} must be int8 or uint8, got {a.dtype}")
    a = a.view(np.uint8)
    if a.size != rows * cols:
        raise ValueError(f"{name} has {a.size} bytes, expected {rows}x{cols}")
    return a.reshape(rows, cols)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p) if a.size else None


def num_threads() -> int:
    """OpenMP threads the oracle's row loop uses."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for later calls (for timing; results do not depend on it)."""
    _load().oracle_set_num_threads(int(n))


def unpack_int4(packed, K: int) -> np.ndarray:
    """Packed bytes [rows, K/2] -> logical int4 values as int8 [rows, K]."""
    p = np.ascontiguousarray(packed)
    rows = p.shape[0] if p.ndim == 2 else 1
    if K % 2:
        raise ValueError("K must be even")
    p = _bytes2d(p, rows, K // 2, "packed")
    out = np.empty((rows, K), dtype=np.int8)
    _check(_load().oracle_unpack_int4(_ptr(p), rows, K, _ptr(out)), "unpack_int4")
    return out


def pack_int4(logical) -> np.ndarray:
    """Logical int4 held as int8 [rows, K] -> packed uint8 [rows, K/2].

    Mirrors the page's packer: int8 input only (TypeError otherwise), last
    dimension even (ValueError otherwise).
    """
    x = np.asarray(logical)
    if x.dtype != np.int8:
        raise TypeError("pack_int4 expects int8 logical values")
    if x.ndim == 0 or x.shape[-1] % 2:
        raise ValueError("the last dimension of a logical int4 tensor must be even")
    K = x.shape[-1]
    rows = x.size // K if K else int(np.prod(x.shape[:-1]))
    x2 = np.ascontiguousarray(x).reshape(rows, K)
    out = np.empty((rows, K // 2), dtype=np.uint8)
    _check(_load().oracle_pack_int4(_ptr(x2), rows, K, _ptr(out)), "pack_int4")
    return out.reshape(x.shape[:-1] + (K // 2,))


def gemm_i4i4(A_packed, B_packed, M: int, N: int, K: int) -> np.ndarray:
    """int4 x int4: C[M,N] int32 = A . B^T from packed [M,K/2] and [N,K/2]."""
    if K % 2 or min(M, N, K) < 0:
        raise ValueError("need M, N, K >= 0 and K even")
    a = _bytes2d(A_packed, M, K // 2, "A_packed")
    b = _bytes2d(B_packed, N, K // 2, "B_packed")
    C = np.zeros((M, N), dtype=np.int32)
    _check(_load().oracle_gemm_i4i4(_ptr(a), _ptr(b), M, N, K, _ptr(C)), "gemm_i4i4")
    return C


def gemm_w4a8(A, B_packed, M: int, N: int, K: int) -> np.ndarray:
    """W4A8: C[M,N] int32 = A . B^T from int8 A [M,K] and packed B [N,K/2]."""
    if K % 2 or min(M, N, K) < 0:
        raise ValueError("need M, N, K >= 0 and K even")
    a = _bytes2d(A, M, K, "A")
    b = _bytes2d(B_packed, N, K // 2, "B_packed")
    C = np.zeros((M, N), dtype=np.int32)
    _check(_load().oracle_gemm_w4a8(_ptr(a), _ptr(b), M, N, K, _ptr(C)), "gemm_w4a8")
    return C


def _at(fn, a, b, M, N, K, ms, ns, what):
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    if ms.shape != ns.shape:
        raise ValueError("ms and ns must have the same shape")
    out = np.zeros(ms.shape, dtype=np.int32)
    _check(fn(_ptr(a), _ptr(b), M, N, K, _ptr(ms), _ptr(ns), ms.size, _ptr(out)), what)
    return out


def gemm_i4i4_at(A_packed, B_packed, M: int, N: int, K: int, ms, ns) -> np.ndarray:
    """Elements C[ms[i], ns[i]] of the int4 x int4 product, each computed alone."""
    a = _bytes2d(A_packed, M, K // 2, "A_packed")
    b = _bytes2d(B_packed, N, K // 2, "B_packed")
    return _at(_load().oracle_gemm_i4i4_at, a, b, M, N, K, ms, ns, "gemm_i4i4_at")


def gemm_w4a8_at(A, B_packed, M: int, N: int, K: int, ms, ns) -> np.ndarray:
    """Elements C[ms[i], ns[i]] of the W4A8 product, each computed alone."""
    a = _bytes2d(A, M, K, "A")
    b = _bytes2d(B_packed, N, K // 2, "B_packed")
    return _at(_load().oracle_gemm_w4a8_at, a, b, M, N, K, ms, ns, "gemm_w4a8_at")


# Output formats of the scaled epilogue (lpgemm_out_dtype order).
FMT_F32, FMT_BF16, FMT_F16 = 0, 1, 2


def scaled_epilogue(C, scale_a, scale_b, fmt: int) -> np.ndarray:
    """D = out(((float)C * scale_a[m]) * scale_b[n]) as the exact value of each
    rounded result (float64 array); fmt 0 binary32, 1 bfloat16, 2 binary16."""
    C = np.ascontiguousarray(C, dtype=np.int32)
    if C.ndim != 2:
        raise ValueError("C must be 2-D")
    M, N = C.shape
    sa = np.ascontiguousarray(scale_a, dtype=np.float32).reshape(-1)
    sb = np.ascontiguousarray(scale_b, dtype=np.float32).reshape(-1)
    if sa.shape[0] != M or sb.shape[0] != N:
        raise ValueError("scale vectors must have M and N entries")
    out = np.empty((M, N), dtype=np.float64)
    _check(_load().oracle_scaled_epilogue(_ptr(C), _ptr(sa), _ptr(sb), M, N, int(fmt), _ptr(out)),
           "oracle_scaled_epilogue")
    return out


def gemm_scaled(variant: str, A, B_packed, scale_a, scale_b, M: int, N: int, K: int,
                fmt: int) -> np.ndarray:
    """The scaled product: the exact integer GEMM, then the scaled epilogue."""
    C = (gemm_i4i4 if variant == "i4i4" else gemm_w4a8)(A, B_packed, M, N, K)
    return scaled_epilogue(C, scale_a, scale_b, fmt)


def gemm_blockscaled(variant: str, A, B_packed, SFA, SFB, M: int, N: int, K: int, g: int,
                     fmt: int) -> np.ndarray:
    """Per-K-block scaled product (the tutorial's gemm_blockscaled read for
    integer operands): the exact integer partial sum of each block of g k,
    times SFA[m][j] then SFB[n][j], added into a binary32 accumulator in block
    order, then out() to fmt (0 binary32, 1 bfloat16, 2 binary16); returned
    as the exact values (float64 [M, N]).  SFA [M, ceil(K/g)], SFB [N,
    ceil(K/g)] float32; variant "i4i4" (A packed) or "w4a8" (A int8)."""
    if K % 2 or min(M, N, K) < 0 or g < 1:
        raise ValueError("need M, N, K >= 0, K even and g >= 1")
    nb = -(-K // g)
    a = _bytes2d(A, M, K // 2 if variant == "i4i4" else K, "A")
    b = _bytes2d(B_packed, N, K // 2, "B_packed")
    sfa = np.ascontiguousarray(SFA, dtype=np.float32)
    sfb = np.ascontiguousarray(SFB, dtype=np.float32)
    if sfa.size != M * nb or sfb.size != N * nb:
        raise ValueError(f"SFA and SFB must be [{M}, {nb}] and [{N}, {nb}]")
    out = np.zeros((M, N), dtype=np.float64)
    _check(_load().oracle_gemm_blockscaled(0 if variant == "i4i4" else 1, _ptr(a), _ptr(b), _ptr(sfa),
                                           _ptr(sfb), M, N, K, g, int(fmt), _ptr(out)),
           "gemm_blockscaled")
    return out


# ---- fp8 GEMM (the tutorial's gemm_fp8 structure, e4m3 operands) ------------------
def fp8_e4m3_decode(codes) -> np.ndarray:
    """Value of each e4m3 byte (float64; NaN for the NaN codes)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    _check(_load().oracle_fp8_e4m3_decode(_ptr(c), c.size, _ptr(out)), "fp8_e4m3_decode")
    return out


def fp8_e4m3_encode(x) -> np.ndarray:
    """Nearest e4m3 code of each value, ties to even, saturating at +-448."""
    v = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint8)
    _check(_load().oracle_fp8_e4m3_encode(_ptr(v), v.size, _ptr(out)), "fp8_e4m3_encode")
    return out


def gemm_fp8(A, B, M: int, N: int, K: int):
    """(C, Cabs): the exact sums C = A . B^T of the decoded e4m3 operands and the
    sums of the products' magnitudes, float64 [M, N] each."""
    a = _bytes2d(A, M, K, "A")
    b = _bytes2d(B, N, K, "B")
    C = np.zeros((M, N), dtype=np.float64)
    Cabs = np.zeros((M, N), dtype=np.float64)
    _check(_load().oracle_gemm_fp8(_ptr(a), _ptr(b), M, N, K, _ptr(C), _ptr(Cabs)), "gemm_fp8")
    return C, Cabs


def fp8_e5m2_decode(codes) -> np.ndarray:
    """Value of each e5m2 byte (float64; +-inf and NaN for those codes)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    _check(_load().oracle_fp8_e5m2_decode(_ptr(c), c.size, _ptr(out)), "fp8_e5m2_decode")
    return out


def fp8_e5m2_encode(x) -> np.ndarray:
    """Nearest e5m2 code of each value, ties to even, infinity from 61440 on."""
    v = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint8)
    _check(_load().oracle_fp8_e5m2_encode(_ptr(v), v.size, _ptr(out)), "fp8_e5m2_encode")
    return out


def gemm_fp8_e5m2(A, B, M: int, N: int, K: int):
    """(C, Cabs) of decoded e5m2 operands: the exact sums C = A . B^T (as the
    nearest float64) and the sums of the products' magnitudes, [M, N] each."""
    a = _bytes2d(A, M, K, "A")
    b = _bytes2d(B, N, K, "B")
    C = np.zeros((M, N), dtype=np.float64)
    Cabs = np.zeros((M, N), dtype=np.float64)
    _check(_load().oracle_gemm_fp8_e5m2(_ptr(a), _ptr(b), M, N, K, _ptr(C), _ptr(Cabs)),
           "gemm_fp8_e5m2")
    return C, Cabs
