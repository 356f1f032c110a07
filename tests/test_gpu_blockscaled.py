"""Per-K-block scaled product on the GPU against the oracle (needs an MI355X).

The reading of the tutorial's gemm_blockscaled for integer operands fixes
every operation: the exact integer partial C_j of each block of g k, term_j =
((float)C_j * SFA[m][j]) * SFB[n][j], the terms added in block order into a
binary32 accumulator, every step rounding to nearest even, then out().  The
result is unique, so the GPU output is decoded to exact values and must equal
the oracle's bit for bit, signs of zeros included, for every kernel (the
one-thread-per-element kernel and the tiled matrix-core kernel with 128- and
64-tiles), every g (32 and 64 have their own fragment maps and flush
schedules, 128 and up share one), every output format, ragged shapes (K not a
multiple of g or of 64, partial tiles) and K = 0.  D sits between guard bands
pre-filled with a sentinel.
"""
import sys

import numpy as np
import pytest

import oracle
import precision_integer_gemm_amd as L
from precision_integer_gemm_amd.inputs import block_scale_table, custom_operands

pytestmark = pytest.mark.gpu

GUARD = 512


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
KERNELS = {"general": L.KERNEL_GENERAL, "t128": L.KERNEL_TILED_128, "t64": L.KERNEL_TILED_64,
           "auto": L.KERNEL_AUTO}


def decode(bits, fmt):
    if fmt == "f32":
        return bits.view(np.float32).astype(np.float64)
    if fmt == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def run_bs(torch, variant, A, B, sfa, sfb, g, M, N, K, fmt, kernel=L.KERNEL_AUTO):
    dev = torch.device("cuda:0")
    a_t = torch.from_numpy(np.ascontiguousarray(A).view(np.uint8).reshape(-1)).to(dev)
    b_t = torch.from_numpy(np.ascontiguousarray(B).reshape(-1)).to(dev)
    sa_t = torch.from_numpy(np.ascontiguousarray(sfa, dtype=np.float32).reshape(-1)).to(dev)
    sb_t = torch.from_numpy(np.ascontiguousarray(sfb, dtype=np.float32).reshape(-1)).to(dev)
    elem = np.uint32 if fmt == "f32" else np.uint16
    tdt = torch.int32 if fmt == "f32" else torch.int16
    sentinel = 0x7EADBEEF if fmt == "f32" else 0x7EAD
    dbuf = torch.full((M * N + 2 * GUARD,), sentinel, dtype=tdt, device=dev)
    d_t = dbuf[GUARD:GUARD + M * N]
    L.lpgemm_set_kernel_override(kernel)
    fn = L.lib().lpgemm_int4_int4_blockscaled if variant == "i4i4" else L.lib().lpgemm_w4a8_blockscaled
    st = fn(a_t.data_ptr(), b_t.data_ptr(), sa_t.data_ptr(), sb_t.data_ptr(), g, d_t.data_ptr(),
            FORMATS[fmt][0], M, N, K, torch.cuda.current_stream().cuda_stream)
    assert st == L.OK, L.lpgemm_status_string(st)
    torch.cuda.synchronize()
    host = dbuf.cpu().numpy().view(elem)
    s = np.array(sentinel, dtype=elem)
    assert (host[:GUARD] == s).all(), "write before D"
    assert (host[GUARD + M * N:] == s).all(), "write after D"
    return decode(host[GUARD:GUARD + M * N], fmt).reshape(M, N)


def check(got, want):
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    same &= np.signbit(got) == np.signbit(want)
    bad = np.argwhere(~same)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:3].tolist()}: " \
                          f"{got[tuple(bad[0])]!r} vs {want[tuple(bad[0])]!r}"


def case(variant, M, N, K, g, seed):
    A, B = custom_operands(variant, M, N, K, seed)
    sfa = block_scale_table(seed, 0, M, K, g)
    sfb = block_scale_table(seed, 1, N, K, g)
    return A, B, sfa, sfb


SHAPES = [(1, 1, 32), (17, 33, 96), (64, 64, 128), (129, 255, 544), (300, 260, 1056), (96, 200, 4128)]


@pytest.mark.parametrize("fmt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("g", [32, 64, 128, 256])
@pytest.mark.parametrize("kernel", ["t128", "t64", "general"])
@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_blockscaled_parity(torch, variant, kernel, g, fmt, M, N, K):
    say(f"blockscaled {variant} {kernel} g={g} {fmt} {M}x{N}x{K}")
    A, B, sfa, sfb = case(variant, M, N, K, g, seed=M + 3 * N + K + g)
    want = oracle.gemm_blockscaled(variant, A, B, sfa, sfb, M, N, K, g, FORMATS[fmt][1])
    check(run_bs(torch, variant, A, B, sfa, sfb, g, M, N, K, fmt, KERNELS[kernel]), want)


@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
@pytest.mark.parametrize("M,N,K,g", [(33, 40, 30, 32), (20, 24, 222, 64), (5, 7, 2, 32)])
def test_ragged_k_takes_the_general_kernel(torch, variant, M, N, K, g):
    # K % 32 != 0: only the one-thread kernel; every block but the last full
    say(f"blockscaled ragged {variant} {M}x{N}x{K} g={g}")
    A, B, sfa, sfb = case(variant, M, N, K, g, seed=7 + K)
    want = oracle.gemm_blockscaled(variant, A, B, sfa, sfb, M, N, K, g, oracle.FMT_F32)
    check(run_bs(torch, variant, A, B, sfa, sfb, g, M, N, K, "f32"), want)


@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
def test_one_block_equals_the_per_channel_product(torch, variant):
    # g >= K: the per-channel scaled entry point's result, bit for bit
    M, N, K = 200, 136, 512
    say(f"blockscaled one block {variant}")
    A, B, sfa, sfb = case(variant, M, N, K, 1024, seed=11)
    got = run_bs(torch, variant, A, B, sfa, sfb, 1024, M, N, K, "bf16")
    dev = torch.device("cuda:0")
    a = torch.from_numpy(np.ascontiguousarray(A)).to(dev)
    b = torch.from_numpy(np.ascontiguousarray(B)).to(dev)
    sa = torch.from_numpy(np.ascontiguousarray(sfa.reshape(-1))).to(dev)
    sb = torch.from_numpy(np.ascontiguousarray(sfb.reshape(-1))).to(dev)
    if variant == "i4i4":
        d = L.lpgemm_int4_int4_scaled(a, b, sa, sb, dtype=torch.bfloat16)
    else:
        d = L.lpgemm_w4a8_scaled(a.view(torch.int8), b, sa, sb, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    check(got, d.float().cpu().numpy().astype(np.float64))


def test_signed_zero_and_block_order(torch):
    # the hand-worked cases of the oracle's pins, on every kernel: partials 1,
    # 2048, 1 with SFA 1, 2^13, 1 give 2^24 (block order); an all-zero row
    # with negative scales gives -0 in every block, so -0 overall
    g, M, N = 64, 64, 64
    K = 3 * g
    a = np.zeros((M, K), np.int8); b = np.zeros((N, K), np.int8)
    a[0, 0] = b[0, 0] = 1
    a[0, g:g + 32] = -8; b[0, g:g + 32] = -8
    a[0, 2 * g] = b[0, 2 * g] = 1
    A, B = oracle.pack_int4(a), oracle.pack_int4(b)
    sfa = np.ones((M, 3), np.float32); sfa[0, 1] = 2.0 ** 13
    sfb = -np.ones((N, 3), np.float32); sfb[0] = 1.0
    want = oracle.gemm_blockscaled("i4i4", A, B, sfa, sfb, M, N, K, g, oracle.FMT_F32)
    assert want[0, 0] == 2.0 ** 24 and np.signbit(want[1, 1])
    for kernel in ("t128", "t64", "general"):
        say(f"blockscaled hand-worked {kernel}")
        check(run_bs(torch, "i4i4", A, B, sfa, sfb, g, M, N, K, "f32", KERNELS[kernel]), want)


def test_k_zero_and_argument_errors(torch):
    say("blockscaled K = 0 and argument errors")
    got = run_bs(torch, "i4i4", np.zeros((3, 0), np.uint8), np.zeros((5, 0), np.uint8),
                 np.zeros((3, 0), np.float32), np.zeros((5, 0), np.float32), 32, 3, 5, 0, "f32")
    assert (got == 0).all() and not np.signbit(got).any()
    dev = torch.device("cuda:0")
    buf = torch.zeros(4096, dtype=torch.int32, device=dev)
    p = buf.data_ptr()
    s = torch.cuda.current_stream().cuda_stream
    fn = L.lib().lpgemm_int4_int4_blockscaled
    assert fn(p, p, p, p, 48, p, L.OUT_F32, 4, 4, 64, s) == L.ERR_INVALID_ARG       # g not a power of two
    assert fn(p, p, p, p, 16, p, L.OUT_F32, 4, 4, 64, s) == L.ERR_INVALID_ARG       # g below 32
    assert fn(p, p, p, p, 32, p, L.OUT_FP8_E4M3, 4, 4, 64, s) == L.ERR_INVALID_ARG
    assert fn(p, p, p, p, 32, p, L.OUT_F32, 4, 4, 63, s) == L.ERR_INVALID_ARG       # odd K
    assert fn(p, p, None, p, 32, p, L.OUT_F32, 4, 4, 64, s) == L.ERR_INVALID_ARG
    assert fn(p, p, p + 2, p, 32, p, L.OUT_F32, 4, 4, 64, s) == L.ERR_INVALID_ARG   # misaligned SFA
    assert fn(p, p, p, p, 32, p + 2, L.OUT_F32, 4, 4, 64, s) == L.ERR_INVALID_ARG   # misaligned D
    assert fn(p, p, p, p, 32, p, L.OUT_F32, 4, 4, L.MAX_K + 2, s) == L.ERR_UNSUPPORTED   # even, too long
    L.lpgemm_set_kernel_override(L.KERNEL_SKINNY)
    assert fn(p, p, p, p, 32, p, L.OUT_F32, 4, 4, 64, s) == L.ERR_UNSUPPORTED
    L.lpgemm_set_kernel_override(L.KERNEL_TILED_128)
    assert fn(p, p, p, p, 32, p, L.OUT_F32, 4, 4, 48, s) == L.ERR_UNSUPPORTED      # K % 32 != 0


@pytest.mark.parametrize("fmt", ["bf16", "f32"])
@pytest.mark.parametrize("variant,M,N,K,g", [("i4i4", 2048, 2048, 4096, 128), ("w4a8", 2048, 2048, 4096, 32),
                                             ("w4a8", 16, 4096, 8192, 128)])
def test_large_shapes_full_parity(torch, variant, M, N, K, g, fmt):
    # automatic kernel choice, every element against the oracle
    say(f"blockscaled large {variant} {M}x{N}x{K} g={g} {fmt}")
    A, B, sfa, sfb = case(variant, M, N, K, g, seed=21)
    want = oracle.gemm_blockscaled(variant, A, B, sfa, sfb, M, N, K, g, FORMATS[fmt][1])
    check(run_bs(torch, variant, A, B, sfa, sfb, g, M, N, K, fmt), want)


def test_tensor_wrappers(torch):
    say("blockscaled tensor wrappers")
    dev = torch.device("cuda:0")
    M, N, K, g = 40, 72, 256, 64
    A, B, sfa, sfb = case("w4a8", M, N, K, g, seed=5)
    want = oracle.gemm_blockscaled("w4a8", A, B, sfa, sfb, M, N, K, g, oracle.FMT_F16)
    d = L.lpgemm_w4a8_blockscaled(torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev),
                                  torch.from_numpy(sfa).to(dev), torch.from_numpy(sfb).to(dev), g,
                                  dtype=torch.float16)
    torch.cuda.synchronize()
    check(d.float().cpu().numpy().astype(np.float64), want)
    with pytest.raises(ValueError):
        L.lpgemm_w4a8_blockscaled(torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev),
                                  torch.from_numpy(sfa[:, :1].copy()).to(dev), torch.from_numpy(sfb).to(dev), g)


@pytest.mark.parametrize("kernel", ["t128", "t64", "general"])
@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
def test_tiny_scales_and_long_blocks(torch, variant, kernel):
    # the tiled kernel folds 2^-shift into SFA only where that is exact: here
    # some SFA rows sit at or below 2^-118 (subnormal once folded, or
    # subnormal already), and g = 2048 lets a block's partial exceed what a
    # folded conversion keeps exact; every such wave must take the unfolded
    # path and still match the oracle bit for bit (subnormal results included)
    M, N, K = 96, 80, 4160
    for g, seed in ((2048, 31), (64, 32), (32, 33)):
        say(f"blockscaled tiny scales {variant} {kernel} g={g}")
        A, B, sfa, sfb = case(variant, M, N, K, g, seed)
        sfa[5] = np.float32(2.0 ** -125)
        sfa[37] = np.float32(3 * 2.0 ** -140)              # subnormal
        sfa[70, :] = np.float32(-1.5 * 2.0 ** -119)
        sfb[3] = np.float32(2.0 ** -20)                    # products into the subnormal range
        want = oracle.gemm_blockscaled(variant, A, B, sfa, sfb, M, N, K, g, oracle.FMT_F32)
        assert (np.abs(want[37]) < 2.0 ** -126).any() or (want[37] == 0).all()
        check(run_bs(torch, variant, A, B, sfa, sfb, g, M, N, K, "f32", KERNELS[kernel]), want)
