"""fp8 GEMM with e5m2 operands on the GPU against the oracle (needs an MI355X).

The tutorial's gemm_fp8 takes either 8-bit format ("e4m3 / e5m2") into a
float32 accumulator.  Comparisons as for e4m3:
  * exact: small-integer operands and sums of identical terms, where no
    summation order or internal alignment rounds, bit for bit, and the e5m2
    rounding of the exact sum;
  * bounded: full-range and adversarial operands.  The one-thread-per-element
    kernel adds exact products in binary32 in k order (within
    1.01 K 2^-24 sum|a b|).  The matrix-core instruction with e5m2 operands
    was measured on MI355X to follow the same summation as with e4m3: groups
    of 8 consecutive k, every product truncated toward zero to a multiple of
    2^(E - 13), E the largest exponent sum of the group's nonzero products (e
    of a subnormal e5m2 code is -14), group sums and accumulator added in
    binary32 round-to-nearest-even; every one of 4 x 4096 single-group cases
    (full exponent range, mid range, subnormals, narrow range) matched that
    model exactly, and no other grid step did.  Hence
        |C - S| <= 7 sum_groups 2^(E_A + E_B - 13) + 1.01 K 2^-24 sum|a b|.
  * special values: e5m2 has infinities; a product with an infinite operand is
    infinite (NaN against zero), opposite infinities give NaN, a NaN operand
    gives NaN, as in IEEE arithmetic and the oracle's double sum.
An e5m2 result must be the rounding of a value in the allowed interval
(round to nearest even, magnitudes from 61440 to infinity).  C sits between
guard bands pre-filled with a sentinel.
"""
import sys

import numpy as np
import pytest

import oracle
import precision_integer_gemm_amd as L
from precision_integer_gemm_amd.inputs import random_bytes
from fp8_bounds import group_exponent_bound

pytestmark = pytest.mark.gpu

GUARD = 1024
U = 2.0 ** -24
INF, NINF, NAN = 0x7C, 0xFC, 0x7F


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    L.lib()
    return t


@pytest.fixture(autouse=True)
def _auto_kernel():
    yield
    L.lpgemm_set_kernel_override(L.KERNEL_AUTO)


def codes(stream, rows, K):
    """Seeded finite e5m2 codes (infinity and NaN codes, exponent field 31,
    moved to the largest finite binade)."""
    c = random_bytes(stream, rows * K)
    c = np.where((c & 0x7C) == 0x7C, c & 0xFB, c).astype(np.uint8)
    return c.reshape(rows, K)


def run_gpu(torch, A, B, M, N, K, fp8_out, kernel=L.KERNEL_AUTO, c_offset=0):
    dev = torch.device("cuda:0")
    a_t = torch.from_numpy(np.ascontiguousarray(A).reshape(-1)).to(dev)
    b_t = torch.from_numpy(np.ascontiguousarray(B).reshape(-1)).to(dev)
    if fp8_out:
        cbuf = torch.full((M * N + 2 * GUARD + c_offset,), 0x5A, dtype=torch.uint8, device=dev)
        c_t = cbuf[GUARD + c_offset:GUARD + c_offset + M * N]
    else:
        cbuf = torch.full((M * N + 2 * GUARD,), 0x7EADBEEF, dtype=torch.int32, device=dev)
        c_t = cbuf[GUARD:GUARD + M * N]
    L.lpgemm_set_kernel_override(kernel)
    st = L.lib().lpgemm_fp8_e5m2(a_t.data_ptr(), b_t.data_ptr(), c_t.data_ptr(),
                                 L.OUT_FP8_E5M2 if fp8_out else L.OUT_F32, M, N, K,
                                 torch.cuda.current_stream().cuda_stream)
    assert st == L.OK, L.lpgemm_status_string(st)
    torch.cuda.synchronize()
    host = cbuf.cpu().numpy()
    lo, hi = GUARD + c_offset, GUARD + c_offset + M * N
    sentinel = 0x5A if fp8_out else 0x7EADBEEF
    assert (host[:lo] == sentinel).all(), "write before C"
    assert (host[hi:] == sentinel).all(), "write after C"
    out = host[lo:hi].reshape(M, N)
    return out if fp8_out else out.view(np.float32).astype(np.float64)


def tolerance(C, Cabs, K, mfma, A=None, B=None):
    tol = 1.01 * K * U * Cabs
    return tol + group_exponent_bound(A, B, K, "e5m2") if mfma else tol


def check_f32(got, C, Cabs, K, mfma=True, A=None, B=None):
    tol = tolerance(C, Cabs, K, mfma, A, B)
    bad = np.argwhere(~(np.abs(got - C) <= tol))
    assert bad.size == 0, f"{len(bad)} outside the bound, first {bad[:3].tolist()}: " \
                          f"{got[tuple(bad[0])]} vs {C[tuple(bad[0])]} (tol {tol[tuple(bad[0])]})"


def check_e5m2(got, C, Cabs, K, mfma=True, A=None, B=None):
    tol = tolerance(C, Cabs, K, mfma, A, B)
    lo = oracle.fp8_e5m2_decode(oracle.fp8_e5m2_encode(C - tol))
    hi = oracle.fp8_e5m2_decode(oracle.fp8_e5m2_encode(C + tol))
    v = oracle.fp8_e5m2_decode(got)
    bad = np.argwhere(~((v >= lo) & (v <= hi)))
    assert bad.size == 0, f"{len(bad)} codes outside the rounding interval, first {bad[:3].tolist()}"


SHAPES = [(1, 1, 16), (17, 33, 48), (37, 53, 96), (129, 255, 512), (300, 260, 1056),
          (513, 257, 2064), (64, 700, 4096)]
RAGGED = [(1, 1, 1), (3, 5, 7), (17, 33, 50), (40, 30, 333)]
TILED = [L.KERNEL_TILED_64, L.KERNEL_TILED_128, L.KERNEL_TILED_256]


@pytest.mark.parametrize("fp8_out", [False, True], ids=["f32", "e5m2"])
@pytest.mark.parametrize("tile", TILED, ids=["t64", "t128", "t256"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_tiled(torch, M, N, K, tile, fp8_out):
    say(f"e5m2 tiled {tile} {M}x{N}x{K} e5m2-out={fp8_out}")
    A, B = codes(M * 3 + K + 50, M, K), codes(N * 5 + K + 51, N, K)
    C, Cabs = oracle.gemm_fp8_e5m2(A, B, M, N, K)
    got = run_gpu(torch, A, B, M, N, K, fp8_out, kernel=tile)
    (check_e5m2 if fp8_out else check_f32)(got, C, Cabs, K, A=A, B=B)


@pytest.mark.parametrize("fp8_out", [False, True], ids=["f32", "e5m2"])
@pytest.mark.parametrize("M,N,K", RAGGED + SHAPES[:4])
def test_general(torch, M, N, K, fp8_out):
    say(f"e5m2 general {M}x{N}x{K} e5m2-out={fp8_out}")
    A, B = codes(M + 7 * K + 60, M, K), codes(N + 11 * K + 61, N, K)
    C, Cabs = oracle.gemm_fp8_e5m2(A, B, M, N, K)
    got = run_gpu(torch, A, B, M, N, K, fp8_out, kernel=L.KERNEL_GENERAL)
    (check_e5m2 if fp8_out else check_f32)(got, C, Cabs, K, mfma=False)


def test_every_code_decodes_and_every_product_encodes(torch):
    # K = 1 runs the one-thread-per-element kernel: C[m][n] is the product of
    # codes m and n, exact in binary32, so the fp32 result is the oracle's
    # product for all 256 x 256 pairs (infinities and NaNs included) and the
    # e5m2 result the oracle's rounding of it
    say("e5m2 all code pairs")
    ALL = np.arange(256, dtype=np.uint8).reshape(256, 1)
    C, _ = oracle.gemm_fp8_e5m2(ALL, ALL, 256, 256, 1)
    got = run_gpu(torch, ALL, ALL, 256, 256, 1, False)
    assert np.array_equal(np.isnan(got), np.isnan(C))
    ok = ~np.isnan(C)
    assert np.array_equal(got[ok], C[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(C[ok]))
    got8 = run_gpu(torch, ALL, ALL, 256, 256, 1, True)
    want8 = oracle.fp8_e5m2_encode(C)
    assert np.array_equal(got8[ok], want8[ok])
    assert ((got8[~ok] & 0x7F) > 0x7C).all()                  # a NaN code


def integer_codes(stream, rows, K):
    """Seeded e5m2 codes of the integers -8 .. 8 (all representable)."""
    v = (random_bytes(stream, rows * K) % 17).astype(np.float64) - 8.0
    return oracle.fp8_e5m2_encode(v).reshape(rows, K)


@pytest.mark.parametrize("kernel", TILED + [L.KERNEL_GENERAL], ids=["t64", "t128", "t256", "general"])
@pytest.mark.parametrize("M,N,K", [(37, 53, 96), (300, 260, 1056), (64, 100, 8192)])
def test_integer_operands_are_exact(torch, M, N, K, kernel):
    # products of magnitude <= 64: E <= 6, the in-group grid step 2^(E - 13)
    # is below 1 and nothing is truncated; |partial sums| <= 64 K are exact
    say(f"e5m2 integer operands {kernel} {M}x{N}x{K}")
    A, B = integer_codes(M + K + 70, M, K), integer_codes(N + 3 * K + 71, N, K)
    C, _ = oracle.gemm_fp8_e5m2(A, B, M, N, K)
    assert np.array_equal(run_gpu(torch, A, B, M, N, K, False, kernel=kernel), C)
    assert np.array_equal(run_gpu(torch, A, B, M, N, K, True, kernel=kernel), oracle.fp8_e5m2_encode(C))


@pytest.mark.parametrize("kernel", [L.KERNEL_AUTO, L.KERNEL_GENERAL], ids=["auto", "general"])
def test_closed_forms_are_exact(torch, kernel):
    M, N, K = 96, 80, 4096
    say(f"e5m2 closed forms kernel {kernel}")
    ones = np.full((M, K), 0x3C, np.uint8)                 # 1.0
    assert (run_gpu(torch, ones, ones[:N], M, N, K, False, kernel=kernel) == K).all()
    # 57344 * -57344 = -49 * 2^26 per term; partial sums 49 j 2^26 are exact
    big, nbig = np.full((M, K), 0x7B, np.uint8), np.full((N, K), 0xFB, np.uint8)
    assert (run_gpu(torch, big, nbig, M, N, K, False, kernel=kernel) == -49.0 * 2.0 ** 38).all()
    # an e5m2 result beyond 61440 overflows to -infinity
    assert (run_gpu(torch, big, nbig, M, N, K, True, kernel=kernel) == NINF).all()
    # 2^-12 * 2^-12 * 4096 = 2^-12 (code 0x0C); 2^-12 * 2^-12 * 256 = 2^-16,
    # the smallest subnormal (code 0x01)
    small = np.full((M, K), 0x0C, np.uint8)
    assert (run_gpu(torch, small, small[:N], M, N, K, True, kernel=kernel) == 0x0C).all()
    assert (run_gpu(torch, small[:, :256], small[:N, :256], M, N, 256, True, kernel=kernel) == 0x01).all()


@pytest.mark.parametrize("kernel", TILED + [L.KERNEL_GENERAL], ids=["t64", "t128", "t256", "general"])
def test_infinities_and_nans(torch, kernel):
    # rows of A with special codes at seeded positions, against the oracle's
    # double sum: finite outputs within the bound, infinite ones with the same
    # sign, NaN where the oracle has NaN
    M, N, K = 64, 48, 256
    say(f"e5m2 infinities kernel {kernel}")
    A, B = codes(81, M, K), codes(82, N, K)
    rng = np.random.default_rng(83)
    for m in range(0, M, 4):
        A[m, rng.integers(0, K)] = [INF, NINF, NAN][m % 3]
    A[1, 5], A[1, 200] = INF, NINF                         # opposite infinities, two groups
    A[2, 9], A[2, 10] = INF, NINF                          # the same group
    B[3, :] = np.where(np.arange(K) % 2 == 0, 0, B[3, :])  # zeros against the infinities
    C, Cabs = oracle.gemm_fp8_e5m2(A, B, M, N, K)
    got = run_gpu(torch, A, B, M, N, K, False, kernel=kernel)
    assert np.isnan(C).any() and np.isinf(C).any()
    assert np.array_equal(np.isnan(got), np.isnan(C))
    inf = np.isinf(C)
    assert np.array_equal(got[inf], C[inf])
    fin = np.isfinite(C)
    mfma = kernel != L.KERNEL_GENERAL
    tol = tolerance(C, Cabs, K, mfma, A, B)
    assert (np.abs(got[fin] - C[fin]) <= tol[fin]).all()


def test_unaligned_output_takes_the_general_kernel(torch):
    M, N, K = 33, 40, 64
    say("e5m2 unaligned C")
    A, B = codes(91, M, K), codes(92, N, K)
    C, Cabs = oracle.gemm_fp8_e5m2(A, B, M, N, K)
    check_e5m2(run_gpu(torch, A, B, M, N, K, True, c_offset=1), C, Cabs, K, mfma=False)


def test_k_zero_and_argument_errors(torch):
    say("e5m2 k0 and argument errors")
    A, B = np.zeros((5, 0), np.uint8), np.zeros((7, 0), np.uint8)
    assert not run_gpu(torch, A, B, 5, 7, 0, False).any()
    assert not run_gpu(torch, A, B, 5, 7, 0, True).any()
    dev = torch.device("cuda:0")
    buf = torch.zeros(64, dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    fn = L.lib().lpgemm_fp8_e5m2
    p = buf.data_ptr()
    assert fn(p, p, p, L.OUT_FP8_E4M3, 1, 1, 16, s) == L.ERR_INVALID_ARG   # the other format
    assert fn(p, p, p, L.OUT_BF16, 1, 1, 16, s) == L.ERR_INVALID_ARG
    assert fn(p, p, p, L.OUT_F32, -1, 1, 16, s) == L.ERR_INVALID_ARG
    assert fn(p, p, None, L.OUT_F32, 1, 1, 16, s) == L.ERR_INVALID_ARG
    assert fn(p, p, p, L.OUT_F32, 1, 1, L.MAX_K + 1, s) == L.ERR_UNSUPPORTED
    assert L.lib().lpgemm_fp8_e4m3(p, p, p, L.OUT_FP8_E5M2, 1, 1, 16, s) == L.ERR_INVALID_ARG
    L.lpgemm_set_kernel_override(L.KERNEL_FP6)
    assert fn(p, p, p, L.OUT_F32, 1, 1, 16, s) == L.ERR_UNSUPPORTED


@pytest.mark.parametrize("fp8_out", [False, True], ids=["f32", "e5m2"])
def test_full_size_parity(torch, fp8_out):
    # 2048 x 2048 x 4096 in the automatic launch (256-tiles), every element
    M, N, K = 2048, 2048, 4096
    say(f"e5m2 {M}x{N}x{K} plan auto, e5m2-out={fp8_out}")
    A, B = codes(131, M, K), codes(137, N, K)
    C, Cabs = oracle.gemm_fp8_e5m2(A, B, M, N, K)
    got = run_gpu(torch, A, B, M, N, K, fp8_out)
    (check_e5m2 if fp8_out else check_f32)(got, C, Cabs, K, A=A, B=B)


def test_tensor_wrapper(torch):
    say("e5m2 tensor wrapper")
    dev = torch.device("cuda:0")
    M, N, K = 40, 72, 256
    A, B = codes(105, M, K), codes(106, N, K)
    C, Cabs = oracle.gemm_fp8_e5m2(A, B, M, N, K)
    a = torch.from_numpy(A).to(dev).view(torch.float8_e5m2)
    b = torch.from_numpy(B).to(dev).view(torch.float8_e5m2)
    c32 = L.lpgemm_fp8_e5m2(a, b)
    c8 = L.lpgemm_fp8_e5m2(a, b, dtype=torch.float8_e5m2)
    torch.cuda.synchronize()
    check_f32(c32.cpu().numpy().astype(np.float64), C, Cabs, K, A=A, B=B)
    check_e5m2(c8.view(torch.uint8).cpu().numpy(), C, Cabs, K, A=A, B=B)
    with pytest.raises(TypeError):
        L.lpgemm_fp8_e5m2(a, b, dtype=torch.float8_e4m3fn)


# ---- adversarial operands for the matrix-core summation ---------------------------
def _e5m2(vals):
    v = np.asarray(vals, dtype=np.float64)
    c = oracle.fp8_e5m2_encode(v)
    assert np.array_equal(oracle.fp8_e5m2_decode(c), v), "value not representable in e5m2"
    return c


def adversarial(kind, rows, K, seed):
    """Operands (A, B) of `rows` rows each: per group of 8 k one dominant
    product and neighbours chosen to lose the most to truncation."""
    rng = np.random.default_rng(seed)
    a = np.zeros((rows, K)); b = np.zeros((rows, K))
    r = np.arange(rows)
    for g in range(K // 8):
        pos = rng.integers(0, 8, rows) + 8 * g
        if kind == "near_grid":
            # 57344 * 57344 (exponent sum 30, grid 2^17) next to products just
            # under multiples of the grid step (1.75 * 2^17, 1.5 * 2^17, ...)
            a[:, 8 * g:8 * g + 8] = rng.choice([57344.0, -57344.0, 49152.0, -28672.0, 14336.0], (rows, 8))
            b[:, 8 * g:8 * g + 8] = 4.0
            a[r, pos] = rng.choice([57344.0, -57344.0], rows)
            b[r, pos] = 57344.0
        elif kind == "cancel":
            # +P and -P in one group with small terms between them
            a[:, 8 * g:8 * g + 8] = rng.choice([0.4375, -0.875, 1.75, 3.5], (rows, 8))
            b[:, 8 * g:8 * g + 8] = 1.0
            other = 8 * g + (pos - 8 * g + 1 + rng.integers(0, 7, rows)) % 8
            a[r, pos] = 28672.0; b[r, pos] = 320.0
            a[r, other] = -28672.0; b[r, other] = 320.0
        elif kind == "subnormal_max":
            # the largest exponent sum comes from a subnormal operand
            # (2^-16 x 57344 = 0.875, exponent sum -14 + 15 = 1): grid 2^-12
            a[:, 8 * g:8 * g + 8] = rng.choice([2.0 ** -14, 1.5 * 2.0 ** -14, 1.75 * 2.0 ** -13], (rows, 8))
            b[:, 8 * g:8 * g + 8] = rng.choice([2.0 ** -6, 2.0 ** -7, 1.75 * 2.0 ** -6], (rows, 8))
            a[r, pos] = 2.0 ** -16; b[r, pos] = 57344.0
    return _e5m2(a).reshape(rows, K), _e5m2(b).reshape(rows, K)


@pytest.mark.parametrize("kind", ["near_grid", "cancel", "subnormal_max"])
@pytest.mark.parametrize("K", [64, 128, 4096])
@pytest.mark.parametrize("fp8_out", [False, True], ids=["f32", "e5m2"])
def test_adversarial_within_the_derived_bound(torch, kind, K, fp8_out):
    M = N = 96
    say(f"e5m2 adversarial {kind} K={K} e5m2-out={fp8_out}")
    A, B = adversarial(kind, M, K, seed=K + 3 * len(kind))
    B = B[np.random.default_rng(K + 1).permutation(N)]
    C, Cabs = oracle.gemm_fp8_e5m2(A, B, M, N, K)
    got = run_gpu(torch, A, B, M, N, K, fp8_out, kernel=L.KERNEL_TILED_64)
    (check_e5m2 if fp8_out else check_f32)(got, C, Cabs, K, A=A, B=B)
    if not fp8_out:
        err = np.abs(got - C) / tolerance(C, Cabs, K, True, A, B)
        say(f"  largest error / bound: {err.max():.3f}")
