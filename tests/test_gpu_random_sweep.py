"""Seeded random shapes through every entry point and every kernel that
accepts them, bit-exact against the oracle (needs an MI355X).

The named cases in the other parity tests pin chosen shapes; this sweep draws
80 more (M up to 700, N up to 1500, K up to 8192, both operand formats) from a
fixed seed, forces each onto a kernel that takes it (the automatic choice, the
one-thread kernel, the tiled kernel at each tile size, the narrow-M kernel for
up to 64 rows, the FP6 path for int4 x int4), and adds the scaled and
per-K-block scaled products and the fp8 GEMM on integer-valued operands, where
the results are unique as well.
"""
import sys

import numpy as np
import pytest

import oracle
import precision_integer_gemm_amd as L
from precision_integer_gemm_amd.inputs import block_scale_table, custom_operands, scale_vector
from test_gpu_parity import oracle_full, run_gpu

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


KERNELS = {"auto": L.KERNEL_AUTO, "general": L.KERNEL_GENERAL, "t64": L.KERNEL_TILED_64,
           "t128": L.KERNEL_TILED_128, "t256": L.KERNEL_TILED_256, "skinny": L.KERNEL_SKINNY,
           "fp6": L.KERNEL_FP6}


def draw_cases(n=80, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        variant = ["i4i4", "w4a8"][i % 2]
        kernel = list(KERNELS)[rng.integers(0, len(KERNELS))]
        if kernel == "fp6" and variant == "w4a8":
            kernel = "t256"
        M = int(rng.integers(1, 65)) if kernel == "skinny" else int(rng.integers(1, 701))
        N = int(rng.integers(1, 1501))
        if kernel in ("auto", "general") and rng.random() < 0.3:
            K = 2 * int(rng.integers(1, 2049))          # any even K
        else:
            K = 32 * int(rng.integers(1, 257))          # the fast kernels' K % 32 == 0
        cases.append((i, variant, kernel, M, N, K))
    return cases


@pytest.mark.parametrize("i,variant,kernel,M,N,K", draw_cases(),
                         ids=[f"{c[0]}-{c[1]}-{c[2]}-{c[3]}x{c[4]}x{c[5]}" for c in draw_cases()])
def test_random_shape(torch, i, variant, kernel, M, N, K):
    say(f"sweep {i} {variant} {kernel} {M}x{N}x{K}")
    A, B = custom_operands(variant, M, N, K, seed=1000 + i)
    got = run_gpu(torch, variant, A, B, M, N, K, kernel=KERNELS[kernel])
    assert np.array_equal(got, oracle_full(variant, A, B, M, N, K))


def scaled_cases(n=16, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        variant = ["i4i4", "w4a8"][i % 2]
        M, N = int(rng.integers(1, 400)), int(rng.integers(1, 900))
        K = 32 * int(rng.integers(1, 128)) if rng.random() < 0.8 else 2 * int(rng.integers(1, 2000))
        g = int(2 ** rng.integers(5, 10))
        fmt = ["f32", "bf16", "f16"][i % 3]
        out.append((i, variant, M, N, K, g, fmt))
    return out


FMT = {"f32": (L.OUT_F32, oracle.FMT_F32, np.float32), "bf16": (L.OUT_BF16, oracle.FMT_BF16, None),
       "f16": (L.OUT_F16, oracle.FMT_F16, np.float16)}


def to_exact(t, fmt):
    if fmt == "bf16":
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def same(got, want):
    return np.array_equal(got, want) and np.array_equal(np.signbit(got), np.signbit(want))


@pytest.mark.parametrize("i,variant,M,N,K,g,fmt", scaled_cases(),
                         ids=[f"{c[0]}-{c[1]}-{c[2]}x{c[3]}x{c[4]}-g{c[5]}-{c[6]}" for c in scaled_cases()])
def test_random_scaled_and_blockscaled(torch, i, variant, M, N, K, g, fmt):
    say(f"sweep scaled {i} {variant} {M}x{N}x{K} g={g} {fmt}")
    dev = torch.device("cuda:0")
    A, B = custom_operands(variant, M, N, K, seed=2000 + i)
    a = torch.from_numpy(np.ascontiguousarray(A)).to(dev)
    b = torch.from_numpy(np.ascontiguousarray(B)).to(dev)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[fmt]
    # per-row / per-column scales
    sa, sb = scale_vector(2000 + i, 0, M), scale_vector(2000 + i, 1, N)
    sa_t, sb_t = torch.from_numpy(sa).to(dev), torch.from_numpy(sb).to(dev)
    if variant == "i4i4":
        d = L.lpgemm_int4_int4_scaled(a, b, sa_t, sb_t, dtype=tdt)
    else:
        d = L.lpgemm_w4a8_scaled(a.view(torch.int8), b, sa_t, sb_t, dtype=tdt)
    torch.cuda.synchronize()
    assert same(to_exact(d, fmt), oracle.gemm_scaled(variant, A, B, sa, sb, M, N, K, FMT[fmt][1]))
    # per-K-block scales
    sfa, sfb = block_scale_table(3000 + i, 0, M, K, g), block_scale_table(3000 + i, 1, N, K, g)
    sfa_t, sfb_t = torch.from_numpy(sfa).to(dev), torch.from_numpy(sfb).to(dev)
    if variant == "i4i4":
        d = L.lpgemm_int4_int4_blockscaled(a, b, sfa_t, sfb_t, g, dtype=tdt)
    else:
        d = L.lpgemm_w4a8_blockscaled(a.view(torch.int8), b, sfa_t, sfb_t, g, dtype=tdt)
    torch.cuda.synchronize()
    assert same(to_exact(d, fmt), oracle.gemm_blockscaled(variant, A, B, sfa, sfb, M, N, K, g, FMT[fmt][1]))


def fp8_cases(n=12, seed=91):
    rng = np.random.default_rng(seed)
    return [(i, ["e4m3", "e5m2"][i % 2], int(rng.integers(1, 600)), int(rng.integers(1, 900)),
             int(rng.integers(1, 3000))) for i in range(n)]


@pytest.mark.parametrize("i,fmt,M,N,K", fp8_cases(),
                         ids=[f"{c[0]}-{c[1]}-{c[2]}x{c[3]}x{c[4]}" for c in fp8_cases()])
def test_random_fp8_integer_operands(torch, i, fmt, M, N, K):
    # integer values -8..8: nothing is rounded anywhere, so the result is the
    # exact sum, on whichever kernel the shape and alignment choose
    say(f"sweep fp8 {i} {fmt} {M}x{N}x{K}")
    rng = np.random.default_rng(4000 + i)
    enc = oracle.fp8_e4m3_encode if fmt == "e4m3" else oracle.fp8_e5m2_encode
    gemm = oracle.gemm_fp8 if fmt == "e4m3" else oracle.gemm_fp8_e5m2
    A = enc(rng.integers(-8, 9, (M, K)).astype(np.float64)).reshape(M, K)
    B = enc(rng.integers(-8, 9, (N, K)).astype(np.float64)).reshape(N, K)
    dev = torch.device("cuda:0")
    fn = L.lpgemm_fp8_e4m3 if fmt == "e4m3" else L.lpgemm_fp8_e5m2
    c = fn(torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev))
    torch.cuda.synchronize()
    want, _ = gemm(A, B, M, N, K)
    assert np.array_equal(c.cpu().numpy().astype(np.float64), want)
