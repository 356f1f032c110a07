"""Bit-exact parity of the HIP kernels with the CPU oracle (needs an MI355X).

Every case feeds the same seeded bytes to the GPU (through the C-ABI binding)
and to the oracle, and compares every output element (the 8192^3 product
included, against one oracle product computed per test module).  C sits between guard bands pre-filled with a sentinel, so a write outside
[0, M) x [0, N) or an element left unwritten fails the test.
"""
import sys

import numpy as np
import pytest

import oracle
import precision_integer_gemm_amd as L
from precision_integer_gemm_amd.inputs import CASES, custom_operands, operands

pytestmark = pytest.mark.gpu

SENTINEL = 0x7EADBEEF
GUARD = 1024  # int32 elements on each side of C (a multiple of 4: keeps C 16-byte aligned)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    L.lib()  # the HIP library must load; there is no fallback
    return t


@pytest.fixture(autouse=True)
def _auto_kernel():
    yield
    L.lpgemm_set_kernel_override(L.KERNEL_AUTO)


def workspace_for(torch, plan_bytes):
    """A 256-byte aligned device workspace of plan_bytes (pointer, bytes, owner)."""
    if plan_bytes == 0:
        return None, 0, None
    buf = torch.empty(plan_bytes + L.WORKSPACE_ALIGN, dtype=torch.uint8, device="cuda:0")
    skip = (-buf.data_ptr()) % L.WORKSPACE_ALIGN
    return buf.data_ptr() + skip, plan_bytes, buf


def run_gpu(torch, variant, A, B, M, N, K, kernel=L.KERNEL_AUTO, a_offset=0, workspace=None):
    """Run one call through the C ABI; returns C as numpy and checks guards.
    workspace None: the "_ws" entry point with the workspace its plan uses;
    False: the entry point without workspace; an int: that many bytes."""
    dev = torch.device("cuda:0")
    a_t = torch.from_numpy(np.ascontiguousarray(A).view(np.uint8).reshape(-1)).to(dev)
    if a_offset:  # shift A to an unaligned address
        buf = torch.zeros(a_t.numel() + a_offset, dtype=torch.uint8, device=dev)
        buf[a_offset:] = a_t
        a_t = buf[a_offset:]
    b_t = torch.from_numpy(np.ascontiguousarray(B).reshape(-1)).to(dev)
    cbuf = torch.full((M * N + 2 * GUARD,), SENTINEL, dtype=torch.int32, device=dev)
    c_t = cbuf[GUARD:GUARD + M * N]
    L.lpgemm_set_kernel_override(kernel)
    s = torch.cuda.current_stream().cuda_stream
    if workspace is False:
        fn = L.lib().lpgemm_int4_int4 if variant == "i4i4" else L.lib().lpgemm_w4a8
        st = fn(a_t.data_ptr(), b_t.data_ptr(), c_t.data_ptr(), M, N, K, s)
    else:
        if workspace is None:
            v = L.VARIANT_I4I4 if variant == "i4i4" else L.VARIANT_W4A8
            workspace = L.lpgemm_plan(v, M, N, K, a_t.data_ptr(), b_t.data_ptr(),
                                      c_t.data_ptr())["workspace_bytes"] if M and N and K else 0
        ws, nws, _keep = workspace_for(torch, workspace)
        fn = L.lib().lpgemm_int4_int4_ws if variant == "i4i4" else L.lib().lpgemm_w4a8_ws
        st = fn(a_t.data_ptr(), b_t.data_ptr(), c_t.data_ptr(), M, N, K, ws, nws, s)
    assert st == L.OK, L.lpgemm_status_string(st)
    torch.cuda.synchronize()
    host = cbuf.cpu().numpy()
    assert (host[:GUARD] == SENTINEL).all(), "write before C"
    assert (host[GUARD + M * N:] == SENTINEL).all(), "write after C"
    return host[GUARD:GUARD + M * N].reshape(M, N)


def oracle_full(variant, A, B, M, N, K):
    return (oracle.gemm_i4i4 if variant == "i4i4" else oracle.gemm_w4a8)(A, B, M, N, K)


# ---- small and ragged shapes, every kernel that accepts them --------------------
RAGGED = [(1, 1, 2), (3, 5, 2), (17, 33, 34), (37, 53, 86), (129, 255, 510), (5, 7, 66)]
ALIGNED = [(1, 1, 32), (16, 64, 128), (17, 33, 64), (37, 53, 96), (129, 255, 512),
           (130, 200, 160), (256, 256, 256), (300, 260, 1056), (255, 129, 4096),
           (600, 700, 2080), (513, 257, 288)]
SKINNY = [(1, 1, 32), (1, 31, 96), (2, 33, 160), (7, 100, 1056), (16, 1000, 4096),
          (16, 64, 128), (13, 257, 8192)]


@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
@pytest.mark.parametrize("M,N,K", RAGGED + ALIGNED)
def test_general_kernel(torch, variant, M, N, K):
    say(f"general {variant} {M}x{N}x{K}")
    A, B = custom_operands(variant, M, N, K, seed=M * 7 + N)
    got = run_gpu(torch, variant, A, B, M, N, K, kernel=L.KERNEL_GENERAL)
    assert np.array_equal(got, oracle_full(variant, A, B, M, N, K))


@pytest.mark.parametrize("tile", [L.KERNEL_TILED_64, L.KERNEL_TILED_128, L.KERNEL_TILED_256],
                         ids=["t64", "t128", "t256"])
@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
@pytest.mark.parametrize("M,N,K", ALIGNED)
def test_tiled_kernel(torch, variant, M, N, K, tile):
    say(f"tiled {tile} {variant} {M}x{N}x{K}")
    A, B = custom_operands(variant, M, N, K, seed=M * 5 + K)
    got = run_gpu(torch, variant, A, B, M, N, K, kernel=tile)
    assert np.array_equal(got, oracle_full(variant, A, B, M, N, K))


# The FP6 path (int4 x int4 only): tails in every dimension, K from one
# k block to several stages, shapes smaller and larger than one 256-tile.
FP6 = ALIGNED + [(1, 300, 64), (257, 1, 96), (513, 1000, 4160), (1000, 513, 8192),
                 (33, 2100, 2048)]


@pytest.mark.parametrize("M,N,K", FP6)
def test_fp6_kernel(torch, M, N, K):
    say(f"fp6 {M}x{N}x{K}")
    A, B = custom_operands("i4i4", M, N, K, seed=M * 7 + N * 3 + K)
    got = run_gpu(torch, "i4i4", A, B, M, N, K, kernel=L.KERNEL_FP6)
    assert np.array_equal(got, oracle_full("i4i4", A, B, M, N, K))


@pytest.mark.parametrize("variant", ["w4a8", "i4i4"])
@pytest.mark.parametrize("M,N,K", SKINNY)
def test_skinny_kernel(torch, variant, M, N, K):
    say(f"skinny {variant} {M}x{N}x{K}")
    A, B = custom_operands(variant, M, N, K, seed=M * 3 + N)
    got = run_gpu(torch, variant, A, B, M, N, K, kernel=L.KERNEL_SKINNY)
    assert np.array_equal(got, oracle_full(variant, A, B, M, N, K))


# K above 8192 on the narrow-M kernel: equal K ranges, each summed into C by its
# own group of workgroups (C zeroed first, int32 atomic adds), or, when there
# are enough strips, taken in turn by the workgroup that owns a strip
SKINNY_SPLIT = [(1, 257, 8224), (16, 1000, 16384), (13, 2049, 12320), (7, 100, 28672),
                (16, 64, 131040), (16, 8192, 28672), (40, 4200, 12320), (3, 4100, 40000)]


@pytest.mark.parametrize("variant", ["w4a8", "i4i4"])
@pytest.mark.parametrize("M,N,K", SKINNY_SPLIT)
def test_skinny_split_k(torch, variant, M, N, K):
    plan = L.lpgemm_plan(L.VARIANT_W4A8 if variant == "w4a8" else L.VARIANT_I4I4, M, N, K)
    say(f"skinny split-K {variant} {M}x{N}x{K} plan={plan}")
    assert plan["kernel"] == "skinny" and plan["k_chunks"] > 1
    A, B = custom_operands(variant, M, N, K, seed=M * 7 + N + K)
    got = run_gpu(torch, variant, A, B, M, N, K)
    assert np.array_equal(got, oracle_full(variant, A, B, M, N, K))
    # a second call must not add onto the first (C is zeroed by the call itself)
    assert np.array_equal(run_gpu(torch, variant, A, B, M, N, K), got)


# 17..64 rows on the narrow-M kernel (forced): row groups of 16, each over all
# strips, and with K above 8192 also K ranges added into C
SKINNY_ROWS = [(17, 100, 256), (32, 1000, 4096), (40, 257, 1056), (64, 2049, 8192),
               (33, 700, 12320)]


@pytest.mark.parametrize("variant", ["w4a8", "i4i4"])
@pytest.mark.parametrize("M,N,K", SKINNY_ROWS)
def test_skinny_row_groups(torch, variant, M, N, K):
    say(f"skinny row groups {variant} {M}x{N}x{K}")
    A, B = custom_operands(variant, M, N, K, seed=M * 11 + N + K)
    got = run_gpu(torch, variant, A, B, M, N, K, kernel=L.KERNEL_SKINNY)
    assert np.array_equal(got, oracle_full(variant, A, B, M, N, K))


@pytest.mark.parametrize("variant,M,N,K", [("w4a8", 32, 3000, 4096), ("i4i4", 64, 1000, 2048),
                                           ("w4a8", 40, 2000, 12320)])
def test_row_groups_automatic_choice(torch, variant, M, N, K):
    plan = L.lpgemm_plan(L.VARIANT_W4A8 if variant == "w4a8" else L.VARIANT_I4I4, M, N, K)
    say(f"automatic row groups {variant} {M}x{N}x{K} plan={plan}")
    assert plan["kernel"] == "skinny"
    A, B = custom_operands(variant, M, N, K, seed=M * 13 + N + K)
    assert np.array_equal(run_gpu(torch, variant, A, B, M, N, K), oracle_full(variant, A, B, M, N, K))


# 64-tiles too few for two per compute unit with long K: K ranges added into C
TILED_SPLIT = [("i4i4", 80, 512, 32768), ("w4a8", 300, 300, 32768), ("w4a8", 100, 700, 65536),
               ("i4i4", 200, 100, 131040)]


@pytest.mark.parametrize("variant,M,N,K", TILED_SPLIT)
def test_tiled_split_k(torch, variant, M, N, K):
    plan = L.lpgemm_plan(L.VARIANT_W4A8 if variant == "w4a8" else L.VARIANT_I4I4, M, N, K)
    say(f"tiled split-K {variant} {M}x{N}x{K} plan={plan}")
    assert (plan["kernel"], plan["tile_m"]) == ("tiled", 64) and plan["k_chunks"] > 1
    A, B = custom_operands(variant, M, N, K, seed=M * 17 + N + K)
    got = run_gpu(torch, variant, A, B, M, N, K)
    assert np.array_equal(got, oracle_full(variant, A, B, M, N, K))
    assert np.array_equal(run_gpu(torch, variant, A, B, M, N, K), got)  # C zeroed per call
    # a workspace with room for two slices only (two ranges), and none (one range)
    assert np.array_equal(run_gpu(torch, variant, A, B, M, N, K, workspace=2 * M * N * 4), got)
    assert np.array_equal(run_gpu(torch, variant, A, B, M, N, K, workspace=False), got)


# 128-tiles on fewer than two thirds of the compute units with long K: K ranges
# into workspace slices; every element against the oracle (at most 3.2e10
# multiply-adds, a fraction of a second on the host's cores)
TILED_SPLIT_128 = [("i4i4", 128, 16384, 12288), ("w4a8", 96, 20000, 16384), ("i4i4", 72, 17000, 14016)]


@pytest.mark.parametrize("variant,M,N,K", TILED_SPLIT_128)
def test_tiled_split_k_128_tiles(torch, variant, M, N, K):
    plan = L.lpgemm_plan(L.VARIANT_W4A8 if variant == "w4a8" else L.VARIANT_I4I4, M, N, K)
    say(f"tiled split-K 128-tiles {variant} {M}x{N}x{K} plan={plan}")
    assert (plan["kernel"], plan["tile_m"]) == ("tiled", 128) and plan["k_chunks"] > 1
    A, B = custom_operands(variant, M, N, K, seed=M * 19 + N + K)
    got = run_gpu(torch, variant, A, B, M, N, K)
    assert np.array_equal(got, oracle_full(variant, A, B, M, N, K))
    assert np.array_equal(run_gpu(torch, variant, A, B, M, N, K), got)  # C rebuilt per call


@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
def test_unaligned_operand_takes_general_path(torch, variant):
    M, N, K = 40, 72, 256
    say(f"unaligned {variant}")
    A, B = custom_operands(variant, M, N, K, seed=77)
    got = run_gpu(torch, variant, A, B, M, N, K, a_offset=3)
    assert np.array_equal(got, oracle_full(variant, A, B, M, N, K))


@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
def test_closed_form_extremes(torch, variant):
    # all -8 (and A = -128): C = 64 K (i4i4) or 1024 K (w4a8) everywhere
    M, N, K = 160, 144, 4096
    say(f"extremes {variant}")
    B = np.full((N, K // 2), 0x88, dtype=np.uint8)
    if variant == "i4i4":
        A, want = np.full((M, K // 2), 0x88, dtype=np.uint8), 64 * K
    else:
        A, want = np.full((M, K), -128, dtype=np.int8), 1024 * K
    assert (run_gpu(torch, variant, A, B, M, N, K) == want).all()


# The largest K the library accepts: the x16 pre-scale keeps every partial sum
# within int32 (16384 * K < 2^31).  All-extreme operands reach the bound: the
# tiled path at the largest multiple of 32, the general path at K = MAX_K.
@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
@pytest.mark.parametrize("K", [L.MAX_K - L.MAX_K % 32, L.MAX_K], ids=["tiled", "general"])
def test_largest_k_closed_forms(torch, variant, K):
    M, N = 64, 48
    say(f"largest K {variant} K={K}")
    B = np.full((N, K // 2), 0x88, dtype=np.uint8)                        # all -8
    if variant == "i4i4":
        A, want = np.full((M, K // 2), 0x88, dtype=np.uint8), 64 * K        # (-8)(-8)
    else:
        A, want = np.full((M, K), -128, dtype=np.int8), 1024 * K            # (-128)(-8)
    got = run_gpu(torch, variant, A, B, M, N, K)
    assert (got == want).all()
    if variant == "i4i4" and K % 32 == 0:
        # the FP6 path's fp32 accumulator holds 64 K < 2^24 exactly
        assert (run_gpu(torch, variant, A, B, M, N, K, kernel=L.KERNEL_FP6) == want).all()
    if K % 32 == 0:
        # the narrow-M kernel over 16 K ranges added into C
        assert (run_gpu(torch, variant, A[:16], B, 16, N, K, kernel=L.KERNEL_SKINNY) == want).all()
    # mixed signs: b = +7 in odd k, -8 in even k; a = -8 (i4i4) or 127 (w4a8)
    B2 = np.full((N, K // 2), 0x78, dtype=np.uint8)
    if variant == "i4i4":
        want2 = (K // 2) * (64 - 56)
    else:
        A = np.full((M, K), 127, dtype=np.int8)
        want2 = (K // 2) * (127 * -8 + 127 * 7)
    got2 = run_gpu(torch, variant, A, B2, M, N, K)
    assert (got2 == want2).all()
    if variant == "i4i4" and K % 32 == 0:
        assert (run_gpu(torch, variant, A, B2, M, N, K, kernel=L.KERNEL_FP6) == want2).all()
    if K % 32 == 0:
        assert (run_gpu(torch, variant, A[:16], B2, 16, N, K, kernel=L.KERNEL_SKINNY) == want2).all()


@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
def test_k_above_the_limit_is_rejected(torch, variant):
    dev = torch.device("cuda:0")
    buf = torch.zeros(64, dtype=torch.int32, device=dev)
    fn = L.lib().lpgemm_int4_int4 if variant == "i4i4" else L.lib().lpgemm_w4a8
    st = fn(buf.data_ptr(), buf.data_ptr(), buf.data_ptr(), 1, 1, L.MAX_K + 2,
            torch.cuda.current_stream().cuda_stream)
    assert st == L.ERR_UNSUPPORTED


@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
def test_k_zero_writes_zeros_and_empty_is_noop(torch, variant):
    say(f"k0 {variant}")
    empty = np.zeros((5, 0), dtype=np.uint8 if variant == "i4i4" else np.int8)
    got = run_gpu(torch, variant, empty, np.zeros((7, 0), np.uint8), 5, 7, 0)
    assert not got.any()
    dev = torch.device("cuda:0")
    C = torch.full((0, 9), 1, dtype=torch.int32, device=dev)
    fn = L.lpgemm_int4_int4 if variant == "i4i4" else L.lpgemm_w4a8
    A = torch.zeros((0, 16), dtype=torch.int8, device=dev)
    assert fn(A, torch.zeros((9, 16 if variant == "i4i4" else 8), dtype=torch.int8 if variant == "i4i4" else torch.uint8,
                             device=dev), out=C).shape == (0, 9)


def test_deterministic_repeats(torch):
    M, N, K = 300, 260, 1056
    say("determinism")
    A, B = custom_operands("w4a8", M, N, K, seed=5)
    first = run_gpu(torch, "w4a8", A, B, M, N, K)
    for _ in range(9):
        assert np.array_equal(run_gpu(torch, "w4a8", A, B, M, N, K), first)


# ---- the automatic tile choice: small M (one row of 64- or 128-tiles), and ------
# ---- 64-tiles where 128-tiles would leave compute units idle --------------------
AUTO_TILE = [("w4a8", 40, 16400, 2080, 64), ("i4i4", 17, 16448, 1024, 64),
             ("w4a8", 24, 32868, 1024, 128), ("i4i4", 64, 65536, 8192, 128),
             ("w4a8", 100, 28700, 2048, 128), ("w4a8", 128, 65600, 512, 128),
             ("i4i4", 256, 8192, 2048, 64), ("w4a8", 520, 8200, 1024, 128)]


@pytest.mark.parametrize("variant,M,N,K,tile", AUTO_TILE)
def test_automatic_tile_choice(torch, variant, M, N, K, tile):
    v = L.VARIANT_I4I4 if variant == "i4i4" else L.VARIANT_W4A8
    plan = L.lpgemm_plan(v, M, N, K)
    say(f"automatic tile {variant} {M}x{N}x{K} plan={plan}")
    assert (plan["kernel"], plan["tile_m"]) == ("tiled", tile)
    A, B = custom_operands(variant, M, N, K, seed=700 + M)
    got = run_gpu(torch, variant, A, B, M, N, K)
    assert np.array_equal(got, oracle_full(variant, A, B, M, N, K))


# ---- the named workloads at full size, in the launch configuration the ----------
# ---- benchmark times (automatic kernel selection) -------------------------------
FULL = ["i4i4_256", "i4i4_1024", "w4a8_4096", "w4a8_skinny_m16", "w4a8_skinny_m1",
        "i4i4_ragged"]


@pytest.mark.parametrize("name", FULL)
def test_named_case_full_parity(torch, name):
    c = CASES[name]
    say(f"case {name}: {c.variant} {c.M}x{c.N}x{c.K} plan={L.lpgemm_plan(L.VARIANT_I4I4 if c.variant == 'i4i4' else L.VARIANT_W4A8, c.M, c.N, c.K)}")
    A, B = operands(c)
    got = run_gpu(torch, c.variant, A, B, c.M, c.N, c.K)
    want = oracle_full(c.variant, A, B, c.M, c.N, c.K)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("name,kernel", [("i4i4_ragged", L.KERNEL_TILED_256), ("i4i4_1024", L.KERNEL_FP6)],
                         ids=["ragged-int8-256", "1024-fp6"])
def test_named_case_full_parity_other_path(torch, name, kernel):
    # the path the automatic choice does not take for the workload: the
    # ragged case (FP6 automatically) on the int8 256-tile kernel, and the
    # single k group of 1024 (int8 64-tiles automatically) on the FP6 path
    c = CASES[name]
    say(f"case {name} forced kernel {kernel}")
    A, B = operands(c)
    got = run_gpu(torch, c.variant, A, B, c.M, c.N, c.K, kernel=kernel)
    assert np.array_equal(got, oracle_full(c.variant, A, B, c.M, c.N, c.K))


@pytest.fixture(scope="module")
def largest_case():
    # the 8192^3 int4 x int4 workload and its whole oracle product (5.5e11
    # multiply-adds on the host's cores, computed once for the module)
    c = CASES["i4i4_8192"]
    A, B = operands(c)
    say(f"case {c.name}: oracle product on {oracle.num_threads()} threads")
    return c, A, B, oracle_full(c.variant, A, B, c.M, c.N, c.K)


@pytest.mark.parametrize("kernel,ws", [(L.KERNEL_AUTO, None), (L.KERNEL_AUTO, False),
                                       (L.KERNEL_TILED_256, None)],
                         ids=["auto-fp6", "auto-no-workspace", "int8-256"])
def test_largest_case_full_parity(torch, largest_case, kernel, ws):
    c, A, B, want = largest_case
    L.lpgemm_set_kernel_override(kernel)
    say(f"case {c.name}: every element, kernel {kernel} workspace {ws} "
        f"plan={L.lpgemm_plan(L.VARIANT_I4I4, c.M, c.N, c.K, workspace_bytes=0 if ws is False else None)}")
    got = run_gpu(torch, c.variant, A, B, c.M, c.N, c.K, kernel=kernel, workspace=ws)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:4].tolist()}"


# The largest K with a single odd product per output next to partial sums of
# up to 64 (K - 1) = 8386496: the fp32 accumulation of the FP6 path must keep
# the low-order unit, wherever in K the odd product falls (first, middle, last
# 64-k block; either lane half; either nibble).  The int8 kernels and the
# general kernel are checked on the same operands.
ODD_KERNELS = [("fp6", L.KERNEL_FP6, 64, 48), ("tiled256", L.KERNEL_TILED_256, 64, 48),
               ("tiled64", L.KERNEL_TILED_64, 64, 48), ("skinny", L.KERNEL_SKINNY, 16, 48),
               ("auto", L.KERNEL_AUTO, 64, 48)]


@pytest.mark.parametrize("variant", ["i4i4", "w4a8"])
@pytest.mark.parametrize("name,kernel,M,N", ODD_KERNELS, ids=[k[0] for k in ODD_KERNELS])
def test_largest_k_one_odd_term(torch, variant, name, kernel, M, N):
    from closed_forms import odd_term_operands, odd_term_product
    if kernel == L.KERNEL_FP6 and variant != "i4i4":
        pytest.skip("the FP6 path serves int4 x int4 only")
    K = L.MAX_K - L.MAX_K % 32
    say(f"largest K one odd term {variant} {name} {M}x{N}x{K}")
    A, B, p, q = odd_term_operands(variant, M, N, K)
    want = odd_term_product(variant, K, p, q)
    got = run_gpu(torch, variant, A, B, M, N, K, kernel=kernel)
    bad = np.argwhere(got != want)
    assert bad.size == 0, (f"{len(bad)} mismatches, first at {bad[:4].tolist()}: "
                           f"got {got[tuple(bad[0])]}, want {want[tuple(bad[0])]}")
    if variant == "i4i4":
        assert want.max() == 64 * K - 63 == 8386497


def test_general_kernel_one_odd_term_at_max_k(torch):
    from closed_forms import odd_term_operands, odd_term_product
    K = L.MAX_K  # not a multiple of 32: the general kernel
    say(f"general one odd term {K}")
    A, B, p, q = odd_term_operands("i4i4", 12, 12, K)
    got = run_gpu(torch, "i4i4", A, B, 12, 12, K)
    assert np.array_equal(got, odd_term_product("i4i4", K, p, q))


# ---- device pack / unpack ---------------------------------------------------------
def test_device_pack_unpack_match_oracle(torch):
    say("pack/unpack")
    dev = torch.device("cuda:0")
    rows, K = 333, 1030
    packed = custom_operands("i4i4", rows, 1, K, seed=3)[0]
    t = torch.from_numpy(packed).to(dev)
    logical = L.lpgemm_unpack_int4(t)
    torch.cuda.synchronize()
    assert np.array_equal(logical.cpu().numpy(), oracle.unpack_int4(packed, K))
    repacked = L.lpgemm_pack_int4(logical)
    torch.cuda.synchronize()
    assert np.array_equal(repacked.cpu().numpy(), packed)
    allb = np.arange(256, dtype=np.uint8).reshape(1, 256)
    out = L.lpgemm_unpack_int4(torch.from_numpy(allb).to(dev)).cpu().numpy()
    assert np.array_equal(out, oracle.unpack_int4(allb, 512))


def test_fp6_workspace_on_two_streams(torch):
    # Two FP6-path calls in flight on different streams at once, each with its
    # own workspace: neither sees the other's re-encoded operands.
    say("fp6 two streams")
    dev = torch.device("cuda:0")
    shapes = [(640, 768, 4160), (512, 1024, 4096)]
    cases = []
    for i, (M, N, K) in enumerate(shapes):
        A, B = custom_operands("i4i4", M, N, K, seed=900 + i)
        cases.append((M, N, K, A, B, torch.from_numpy(np.ascontiguousarray(A).view(np.uint8)).to(dev),
                      torch.from_numpy(B).to(dev)))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.full((M, N), SENTINEL, dtype=torch.int32, device=dev) for M, N, *_ in cases]
    L.lpgemm_set_kernel_override(L.KERNEL_FP6)
    wss = [workspace_for(torch, L.lpgemm_plan(L.VARIANT_I4I4, M, N, K)["workspace_bytes"])
           for M, N, K, *_ in cases]
    assert all(n > 0 for _, n, _ in wss)
    torch.cuda.synchronize()
    for rep in range(3):
        for (M, N, K, A, B, a_t, b_t), s, c_t, (ws, nws, _) in zip(cases, streams, outs, wss):
            st = L.lib().lpgemm_int4_int4_ws(a_t.data_ptr(), b_t.data_ptr(), c_t.data_ptr(), M, N, K,
                                             ws, nws, s.cuda_stream)
            assert st == L.OK, L.lpgemm_status_string(st)
    torch.cuda.synchronize()
    for (M, N, K, A, B, *_), c_t in zip(cases, outs):
        assert np.array_equal(c_t.cpu().numpy(), oracle_full("i4i4", A, B, M, N, K))
