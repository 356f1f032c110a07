"""Large ragged grids, and shapes with more 256-tiles than workgroups, where
every persistent workgroup walks several tiles (needs an MI355X).

The tiled and FP6 kernels issue a tile's scale vectors (scaled outputs) into
one of two LDS slots with its first copies, and the next tile's first copies
before the current tile's stores.  The 256-tile and FP6 cases here (576 tiles
for 256 workgroups) run that order across tile changes in every output
format: per-row / per-column scaled products, int32 products, and the fp8 GEMM
(both operand formats, binary32 and fp8 output, integer-valued operands so
the result is exact).  The 64- and 128-tile cases (one tile per workgroup)
and the per-K-block scaled cases cover the same epilogue on grids of 288-576
workgroups.  Edges are ragged in M and N, so whole tiles and edge tiles
alternate within a workgroup.  Every element is compared with the oracle.
"""
import sys

import numpy as np
import pytest

import oracle
import precision_integer_gemm_amd as L
from precision_integer_gemm_amd.inputs import custom_operands, scale_vector
from test_gpu_blockscaled import case as bs_case
from test_gpu_blockscaled import check as bs_check
from test_gpu_blockscaled import run_bs
from test_gpu_scaled import FORMATS, check, run_scaled

pytestmark = pytest.mark.gpu


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


# (kernel, M, N, K): 576 and 288 tiles (one per workgroup), then 576 256-tiles
# for 256 persistent workgroups
SCALED = [(L.KERNEL_TILED_64, 2000, 1100, 256), (L.KERNEL_TILED_128, 2000, 2200, 256),
          (L.KERNEL_TILED_256, 6000, 6000, 128), (L.KERNEL_FP6, 6000, 6000, 256)]
_products = {}


def integer_product(variant, M, N, K, seed):
    key = (variant, M, N, K, seed)
    if key not in _products:
        A, B = custom_operands(variant, M, N, K, seed=seed)
        fn = oracle.gemm_i4i4 if variant == "i4i4" else oracle.gemm_w4a8
        _products.clear()
        _products[key] = (A, B, fn(A, B, M, N, K))
    return _products[key]


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
@pytest.mark.parametrize("kernel,M,N,K", SCALED, ids=["t64", "t128", "t256", "fp6"])
def test_scaled_outputs(torch, kernel, M, N, K, variant, fmt):
    if kernel == L.KERNEL_FP6 and variant == "w4a8":
        pytest.skip("the FP6 path takes int4 x int4 only")
    say(f"tile changes scaled {kernel} {variant} {fmt} {M}x{N}x{K}")
    A, B, C = integer_product(variant, M, N, K, seed=M + K)
    sa, sb = scale_vector(M + N, 0, M), scale_vector(M + N, 1, N)
    got = run_scaled(torch, variant, A, B, sa, sb, M, N, K, fmt, kernel=kernel)
    check(got, oracle.scaled_epilogue(C, sa, sb, FORMATS[fmt][1]))


def _run_int32(torch, variant, A, B, M, N, K, kernel):
    from test_gpu_parity import run_gpu
    return run_gpu(torch, variant, A, B, M, N, K, kernel=kernel)


@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
@pytest.mark.parametrize("kernel,M,N,K", SCALED, ids=["t64", "t128", "t256", "fp6"])
def test_int32_output(torch, kernel, M, N, K, variant):
    if kernel == L.KERNEL_FP6 and variant == "w4a8":
        pytest.skip("the FP6 path takes int4 x int4 only")
    say(f"tile changes int32 {kernel} {variant} {M}x{N}x{K}")
    A, B, C = integer_product(variant, M, N, K, seed=M + K)
    assert np.array_equal(_run_int32(torch, variant, A, B, M, N, K, kernel), C)


FP8 = [(L.KERNEL_TILED_64, 2000, 1100, 128), (L.KERNEL_TILED_128, 2000, 2200, 128),
       (L.KERNEL_TILED_256, 6000, 6000, 128)]


@pytest.mark.parametrize("fp8_out", [False, True], ids=["f32", "fp8"])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("kernel,M,N,K", FP8, ids=["t64", "t128", "t256"])
def test_fp8_integer_operands(torch, kernel, M, N, K, fmt, fp8_out):
    # integers -8 .. 8 in either format: products of magnitude <= 64 and
    # partial sums below 2^24, so binary32 results are exact
    if fmt == "e4m3":
        import test_gpu_fp8 as T
        enc = oracle.fp8_e4m3_encode
    else:
        import test_gpu_fp8_e5m2 as T
        enc = oracle.fp8_e5m2_encode
    say(f"tile changes fp8 {fmt} {'fp8' if fp8_out else 'f32'} {kernel} {M}x{N}x{K}")
    A, B = T.integer_codes(M + K, M, K), T.integer_codes(N + 3 * K, N, K)
    av = (oracle.fp8_e4m3_decode if fmt == "e4m3" else oracle.fp8_e5m2_decode)(A)
    bv = (oracle.fp8_e4m3_decode if fmt == "e4m3" else oracle.fp8_e5m2_decode)(B)
    C = av @ bv.T  # exact: integers, |sums| <= 64 K in float64
    got = T.run_gpu(torch, A, B, M, N, K, fp8_out, kernel=kernel)
    assert np.array_equal(got, enc(C) if fp8_out else C)


BLOCK = [("t64", 1100, 1200, 512, 64), ("t128", 2100, 2200, 512, 128), ("t128", 2100, 2200, 512, 32)]


@pytest.mark.parametrize("fmt", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
@pytest.mark.parametrize("kernel,M,N,K,g", BLOCK, ids=["t64-g64", "t128-g128", "t128-g32"])
def test_blockscaled(torch, kernel, M, N, K, g, variant, fmt):
    from test_gpu_blockscaled import FORMATS as BSF
    from test_gpu_blockscaled import KERNELS
    say(f"tile changes block-scaled {kernel} {variant} g={g} {fmt} {M}x{N}x{K}")
    A, B, sfa, sfb = bs_case(variant, M, N, K, g, seed=M + g)
    want = oracle.gemm_blockscaled(variant, A, B, sfa, sfb, M, N, K, g, BSF[fmt][1])
    bs_check(run_bs(torch, variant, A, B, sfa, sfb, g, M, N, K, fmt, kernel=KERNELS[kernel]), want)
