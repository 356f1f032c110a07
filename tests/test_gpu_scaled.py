"""Per-row / per-column scaled output (fp32, bf16, fp16) against the oracle
(needs an MI355X).

Both sides perform the same binary32 operations with round-to-nearest-even
((float)C, then * scale_a[m], then * scale_b[n]) and the same nearest-even
conversion to the output format, so the results must agree bit for bit: the
GPU output is decoded to exact values and compared, signs of zeros included.
The output sits between guard bands pre-filled with a sentinel.
"""
import sys

import numpy as np
import pytest

import oracle
import precision_integer_gemm_amd as L
from precision_integer_gemm_amd.inputs import CASES, custom_operands, operands, scale_vector

pytestmark = pytest.mark.gpu

GUARD = 512  # elements on each side of D (keeps 16-byte alignment for 2- and 4-byte types)


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


FORMATS = {"f32": (L.OUT_F32, oracle.FMT_F32), "bf16": (L.OUT_BF16, oracle.FMT_BF16),
           "f16": (L.OUT_F16, oracle.FMT_F16)}


def decode(bits, fmt):
    """Device output bits -> exact float64 values."""
    if fmt == "f32":
        return bits.view(np.float32).astype(np.float64)
    if fmt == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def run_scaled(torch, variant, A, B, sa, sb, M, N, K, fmt, kernel=L.KERNEL_AUTO):
    dev = torch.device("cuda:0")
    a_t = torch.from_numpy(np.ascontiguousarray(A).view(np.uint8).reshape(-1)).to(dev)
    b_t = torch.from_numpy(np.ascontiguousarray(B).reshape(-1)).to(dev)
    sa_t = torch.from_numpy(np.ascontiguousarray(sa)).to(dev)
    sb_t = torch.from_numpy(np.ascontiguousarray(sb)).to(dev)
    elem = np.uint32 if fmt == "f32" else np.uint16
    tdt = torch.int32 if fmt == "f32" else torch.int16
    sentinel = 0x7EADBEEF if fmt == "f32" else 0x7EAD
    dbuf = torch.full((M * N + 2 * GUARD,), sentinel, dtype=tdt, device=dev)
    d_t = dbuf[GUARD:GUARD + M * N]
    L.lpgemm_set_kernel_override(kernel)
    s = torch.cuda.current_stream().cuda_stream
    if variant == "i4i4":
        # the "_ws" entry point with the workspace the call can use (the FP6
        # path's re-encoded operands; none for the other kernels)
        nws = L.lpgemm_plan(L.VARIANT_I4I4, M, N, K)["workspace_bytes"] if M and N and K else 0
        ws = torch.empty(nws + L.WORKSPACE_ALIGN, dtype=torch.uint8, device=dev)
        ptr = ws.data_ptr() + (-ws.data_ptr()) % L.WORKSPACE_ALIGN if nws else None
        st = L.lib().lpgemm_int4_int4_scaled_ws(a_t.data_ptr(), b_t.data_ptr(), sa_t.data_ptr(),
                                                sb_t.data_ptr(), d_t.data_ptr(), FORMATS[fmt][0],
                                                M, N, K, ptr, nws, s)
    else:
        st = L.lib().lpgemm_w4a8_scaled(a_t.data_ptr(), b_t.data_ptr(), sa_t.data_ptr(),
                                        sb_t.data_ptr(), d_t.data_ptr(), FORMATS[fmt][0], M, N, K, s)
    assert st == L.OK, L.lpgemm_status_string(st)
    torch.cuda.synchronize()
    host = dbuf.cpu().numpy().view(elem)
    assert (host[:GUARD] == elem(sentinel)).all(), "write before D"
    assert (host[GUARD + M * N:] == elem(sentinel)).all(), "write after D"
    return decode(host[GUARD:GUARD + M * N], fmt).reshape(M, N)


def check(got, want):
    bad = np.argwhere(~((got == want) & (np.signbit(got) == np.signbit(want))))
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:4].tolist()}: " \
                          f"{got[tuple(bad[0])]} vs {want[tuple(bad[0])]}"


SHAPES = [(1, 1, 2), (17, 33, 34), (37, 53, 96), (129, 255, 512), (300, 260, 1056),
          (513, 257, 288)]
TILED = [(16, 64, 128), (129, 255, 512), (300, 260, 1056), (600, 700, 2080), (255, 129, 4096)]
SKINNY = [(1, 31, 96), (7, 100, 1056), (16, 1000, 4096), (13, 257, 8192), (40, 300, 1024)]


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_general_kernel(torch, variant, fmt, M, N, K):
    say(f"scaled general {variant} {fmt} {M}x{N}x{K}")
    A, B = custom_operands(variant, M, N, K, seed=M + 3 * N)
    sa, sb = scale_vector(M + N, 0, M), scale_vector(M + N, 1, N)
    got = run_scaled(torch, variant, A, B, sa, sb, M, N, K, fmt, kernel=L.KERNEL_GENERAL)
    check(got, oracle.gemm_scaled(variant, A, B, sa, sb, M, N, K, FORMATS[fmt][1]))


@pytest.mark.parametrize("tile", [L.KERNEL_TILED_64, L.KERNEL_TILED_128, L.KERNEL_TILED_256],
                         ids=["t64", "t128", "t256"])
@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
@pytest.mark.parametrize("M,N,K", TILED)
def test_tiled_kernel(torch, variant, fmt, M, N, K, tile):
    say(f"scaled tiled {tile} {variant} {fmt} {M}x{N}x{K}")
    A, B = custom_operands(variant, M, N, K, seed=2 * M + K)
    sa, sb = scale_vector(M + K, 0, M), scale_vector(M + K, 1, N)
    got = run_scaled(torch, variant, A, B, sa, sb, M, N, K, fmt, kernel=tile)
    check(got, oracle.gemm_scaled(variant, A, B, sa, sb, M, N, K, FORMATS[fmt][1]))


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("M,N,K", TILED)
def test_fp6_kernel(torch, fmt, M, N, K):
    say(f"scaled fp6 {fmt} {M}x{N}x{K}")
    A, B = custom_operands("i4i4", M, N, K, seed=3 * M + K)
    sa, sb = scale_vector(M + 2 * K, 0, M), scale_vector(M + 2 * K, 1, N)
    got = run_scaled(torch, "i4i4", A, B, sa, sb, M, N, K, fmt, kernel=L.KERNEL_FP6)
    check(got, oracle.gemm_scaled("i4i4", A, B, sa, sb, M, N, K, FORMATS[fmt][1]))


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("variant", ["w4a8", "i4i4"])
@pytest.mark.parametrize("M,N,K", SKINNY)
def test_skinny_kernel(torch, variant, fmt, M, N, K):
    say(f"scaled skinny {variant} {fmt} {M}x{N}x{K}")
    A, B = custom_operands(variant, M, N, K, seed=M * 5 + N)
    sa, sb = scale_vector(N, 0, M), scale_vector(N, 1, N)
    got = run_scaled(torch, variant, A, B, sa, sb, M, N, K, fmt, kernel=L.KERNEL_SKINNY)
    check(got, oracle.gemm_scaled(variant, A, B, sa, sb, M, N, K, FORMATS[fmt][1]))


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_narrow_m_long_k_scaled(torch, fmt):
    # K above 8192 with M <= 16: the int32 result would be split over K ranges
    # and added into C; a scaled result cannot be, and takes the tiled kernel
    M, N, K = 16, 300, 9216
    say(f"scaled narrow-M long K {fmt} {M}x{N}x{K}")
    A, B = custom_operands("w4a8", M, N, K, seed=91)
    sa, sb = scale_vector(91, 0, M), scale_vector(91, 1, N)
    got = run_scaled(torch, "w4a8", A, B, sa, sb, M, N, K, fmt)
    check(got, oracle.gemm_scaled("w4a8", A, B, sa, sb, M, N, K, FORMATS[fmt][1]))


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("variant,M,N,K", [("w4a8", 16, 4100, 9216), ("i4i4", 5, 2050, 16448),
                                           ("w4a8", 40, 4200, 12320)])
def test_narrow_m_long_k_ranges_in_turn(torch, variant, fmt, M, N, K):
    # enough strips: each workgroup takes every K range of its strips and
    # stores the sum once, so a scaled result works too
    v = L.VARIANT_W4A8 if variant == "w4a8" else L.VARIANT_I4I4
    assert L.lpgemm_plan(v, M, N, K)["kernel"] == "skinny"
    say(f"scaled narrow-M ranges in turn {variant} {fmt} {M}x{N}x{K}")
    A, B = custom_operands(variant, M, N, K, seed=M + N + K)
    sa, sb = scale_vector(92, 0, M), scale_vector(92, 1, N)
    got = run_scaled(torch, variant, A, B, sa, sb, M, N, K, fmt)
    check(got, oracle.gemm_scaled(variant, A, B, sa, sb, M, N, K, FORMATS[fmt][1]))


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
def test_k_zero_gives_signed_zeros(torch, variant, fmt):
    say(f"scaled k0 {variant} {fmt}")
    M, N = 5, 7
    A = np.zeros((M, 0), dtype=np.uint8 if variant == "i4i4" else np.int8)
    B = np.zeros((N, 0), np.uint8)
    sa, sb = scale_vector(9, 0, M), scale_vector(9, 1, N)
    got = run_scaled(torch, variant, A, B, sa, sb, M, N, 0, fmt)
    check(got, oracle.scaled_epilogue(np.zeros((M, N), np.int32), sa, sb, FORMATS[fmt][1]))


@pytest.mark.parametrize("name", ["w4a8_skinny_m16", "w4a8_skinny_m1", "i4i4_1024", "w4a8_4096"])
def test_named_case_bf16(torch, name):
    c = CASES[name]
    say(f"scaled case {name} bf16")
    A, B = operands(c)
    sa, sb = scale_vector(c.seed, 0, c.M), scale_vector(c.seed, 1, c.N)
    got = run_scaled(torch, c.variant, A, B, sa, sb, c.M, c.N, c.K, "bf16")
    check(got, oracle.gemm_scaled(c.variant, A, B, sa, sb, c.M, c.N, c.K, oracle.FMT_BF16))


def test_largest_case_bf16_rows_and_columns(torch):
    # 8192^3 int4 x int4 in its benchmarked launch (the FP6 path), bf16 output:
    # whole rows and columns against the oracle's integer results and epilogue
    c = CASES["i4i4_8192"]
    say(f"scaled case {c.name} bf16, plan={L.lpgemm_plan(L.VARIANT_I4I4, c.M, c.N, c.K)}")
    A, B = operands(c)
    sa, sb = scale_vector(c.seed, 0, c.M), scale_vector(c.seed, 1, c.N)
    got = run_scaled(torch, c.variant, A, B, sa, sb, c.M, c.N, c.K, "bf16")
    for m in (0, 255, 256, 4097, c.M - 1):
        cm = oracle.gemm_i4i4_at(A, B, c.M, c.N, c.K, np.full(c.N, m), np.arange(c.N))
        want = oracle.scaled_epilogue(cm.reshape(1, c.N).astype(np.int32), sa[m:m + 1], sb,
                                      oracle.FMT_BF16)
        check(got[m:m + 1], want)
    for n in (0, 3, 255, 6001, c.N - 1):
        cn = oracle.gemm_i4i4_at(A, B, c.M, c.N, c.K, np.arange(c.M), np.full(c.M, n))
        want = oracle.scaled_epilogue(cn.reshape(c.M, 1).astype(np.int32), sa, sb[n:n + 1],
                                      oracle.FMT_BF16)
        check(got[:, n:n + 1], want)


def test_tensor_wrappers(torch):
    say("scaled tensor wrappers")
    dev = torch.device("cuda:0")
    M, N, K = 40, 72, 256
    A, B = custom_operands("w4a8", M, N, K, seed=8)
    sa, sb = scale_vector(8, 0, M), scale_vector(8, 1, N)
    d = L.lpgemm_w4a8_scaled(torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev),
                             torch.from_numpy(sa).to(dev), torch.from_numpy(sb).to(dev),
                             dtype=torch.float16)
    torch.cuda.synchronize()
    check(d.cpu().numpy().astype(np.float64),
          oracle.gemm_scaled("w4a8", A, B, sa, sb, M, N, K, oracle.FMT_F16))
