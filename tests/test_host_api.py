"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every entry point include/lpgemm.h declares, rejects bad arguments before any
HIP call, and plans the expected kernel for each shape."""
import ctypes
import os
import re

import numpy as np
import pytest

import precision_integer_gemm_amd as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    with open(os.path.join(ROOT, "include", "lpgemm.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lpgemm_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(L.EXPORTS), names
    raw = ctypes.CDLL(L.LIB_PATH)
    for name in names:
        assert hasattr(raw, name), name


def test_status_strings():
    assert L.lpgemm_status_string(L.OK) == "ok"
    assert L.lpgemm_status_string(L.ERR_INVALID_ARG) == "invalid argument"
    assert L.lpgemm_status_string(L.ERR_UNSUPPORTED) == "unsupported"
    assert L.lpgemm_status_string(L.ERR_HIP) == "HIP runtime error"
    assert L.lpgemm_status_string(99) == "unknown status"


# Arguments rejected on the host: none of these reaches the HIP runtime.
P = 4096  # a fake, 16-byte aligned device address (never dereferenced here)
BAD = [
    ("negative M", (P, P, P, -1, 4, 32), L.ERR_INVALID_ARG),
    ("negative N", (P, P, P, 4, -1, 32), L.ERR_INVALID_ARG),
    ("negative K", (P, P, P, 4, 4, -2), L.ERR_INVALID_ARG),
    ("odd K", (P, P, P, 4, 4, 33), L.ERR_INVALID_ARG),
    ("K above the exact range", (P, P, P, 4, 4, L.MAX_K + 2), L.ERR_UNSUPPORTED),
    ("null C", (P, P, None, 4, 4, 32), L.ERR_INVALID_ARG),
    ("null A", (None, P, P, 4, 4, 32), L.ERR_INVALID_ARG),
    ("null B", (P, None, P, 4, 4, 32), L.ERR_INVALID_ARG),
    ("null C with K = 0", (None, None, None, 4, 4, 0), L.ERR_INVALID_ARG),
]


@pytest.mark.parametrize("fn", ["lpgemm_int4_int4", "lpgemm_w4a8"])
@pytest.mark.parametrize("what,args,want", BAD, ids=[b[0] for b in BAD])
def test_argument_errors(fn, what, args, want):
    a, b, c, M, N, K = args
    assert getattr(L.lib(), fn)(a, b, c, M, N, K, None) == want


@pytest.mark.parametrize("fn", ["lpgemm_int4_int4", "lpgemm_w4a8"])
def test_empty_outputs_are_a_no_op(fn):
    f = getattr(L.lib(), fn)
    assert f(None, None, None, 0, 5, 32, None) == L.OK
    assert f(None, None, None, 5, 0, 32, None) == L.OK


@pytest.mark.parametrize("fn", ["lpgemm_int4_int4_scaled", "lpgemm_w4a8_scaled"])
def test_scaled_argument_errors(fn):
    f = getattr(L.lib(), fn)
    assert f(P, P, P, P, P, 3, 4, 4, 32, None) == L.ERR_INVALID_ARG        # unknown out dtype
    assert f(P, P, None, P, P, L.OUT_BF16, 4, 4, 32, None) == L.ERR_INVALID_ARG  # null scale_a
    assert f(P, P, P, None, P, L.OUT_BF16, 4, 4, 32, None) == L.ERR_INVALID_ARG  # null scale_b
    assert f(P, P, P + 2, P, P, L.OUT_F32, 4, 4, 32, None) == L.ERR_INVALID_ARG  # misaligned scale
    assert f(P, P, P, P, P + 2, L.OUT_F32, 4, 4, 32, None) == L.ERR_INVALID_ARG  # misaligned fp32 D
    assert f(P, P, P, P, P + 1, L.OUT_BF16, 4, 4, 32, None) == L.ERR_INVALID_ARG  # misaligned bf16 D
    assert f(P, P, P, P, None, L.OUT_F16, 4, 4, 32, None) == L.ERR_INVALID_ARG   # null D
    assert f(P, P, P, P, P, L.OUT_F16, 4, 4, 33, None) == L.ERR_INVALID_ARG      # odd K
    assert f(None, None, None, None, None, L.OUT_F16, 0, 4, 32, None) == L.OK    # empty


def test_max_k_is_the_exact_range_of_the_prescale():
    # every x16-scaled term is at most 128*128 = 16384 in magnitude
    assert 16384 * L.MAX_K <= 2**31 - 1 < 16384 * (L.MAX_K + 2)
    assert L.MAX_K % 2 == 0


def test_pack_unpack_argument_errors():
    lib = L.lib()
    assert lib.lpgemm_pack_int4(P, P, 2, 3, None) == L.ERR_INVALID_ARG
    assert lib.lpgemm_pack_int4(P, P, -1, 4, None) == L.ERR_INVALID_ARG
    assert lib.lpgemm_unpack_int4(None, P, 2, 4, None) == L.ERR_INVALID_ARG
    assert lib.lpgemm_unpack_int4(None, None, 0, 4, None) == L.OK
    # rows * K/2 past the int64 range is refused before any HIP call
    assert lib.lpgemm_pack_int4(P, P, 1 << 62, 8, None) == L.ERR_UNSUPPORTED
    assert lib.lpgemm_unpack_int4(P, P, 1 << 62, 8, None) == L.ERR_UNSUPPORTED


def test_kernel_override_rejects_unknown_values():
    with pytest.raises(L.LpgemmError):
        L.lpgemm_set_kernel_override(8)
    with pytest.raises(L.LpgemmError):
        L.lpgemm_set_kernel_override(-1)
    L.lpgemm_set_kernel_override(L.KERNEL_FP6)
    L.lpgemm_set_kernel_override(L.KERNEL_AUTO)


# ---- planning -----------------------------------------------------------------
@pytest.mark.parametrize("variant,M,N,K,kernel", [
    (L.VARIANT_W4A8, 16, 28672, 8192, "skinny"),
    (L.VARIANT_W4A8, 1, 28672, 8192, "skinny"),
    (L.VARIANT_W4A8, 4096, 4096, 4096, "tiled"),
    (L.VARIANT_I4I4, 8192, 8192, 8192, "fp6"),     # 1024 tiles >= 2 x 256 CUs
    (L.VARIANT_I4I4, 3000, 5120, 6144, "fp6"),     # 240 tiles >= 3/4 of the CUs, K >= 3072
    (L.VARIANT_I4I4, 8192, 8192, 2048, "fp6"),     # 1024 tiles, K = 2048
    (L.VARIANT_I4I4, 8192, 8192, 1024, "tiled"),   # K below 2048
    (L.VARIANT_I4I4, 8192, 4096, 4096, "fp6"),     # 512 tiles
    (L.VARIANT_I4I4, 4096, 4096, 4096, "fp6"),     # 256 tiles, K >= 3072
    (L.VARIANT_I4I4, 4096, 4096, 2048, "tiled"),   # 256 tiles, K below 3072
    (L.VARIANT_I4I4, 3840, 4096, 16384, "fp6"),    # 240 tiles
    (L.VARIANT_I4I4, 3072, 3072, 4096, "tiled"),   # 144 tiles: under 3/4 of the CUs
    (L.VARIANT_W4A8, 8192, 8192, 8192, "tiled"),   # FP6 is int4 x int4 only
    (L.VARIANT_I4I4, 256, 256, 256, "tiled"),
    (L.VARIANT_I4I4, 17, 33, 34, "general"),     # K % 32 != 0
    (L.VARIANT_W4A8, 16, 100, 34, "general"),
])
def test_auto_plan(variant, M, N, K, kernel):
    assert L.lpgemm_plan(variant, M, N, K)["kernel"] == kernel


def test_fp6_plan():
    p = L.lpgemm_plan(L.VARIANT_I4I4, 8192, 8192, 8192)
    assert (p["kernel"], p["tile_m"], p["tile_n"], p["workgroups"], p["threads"]) == ("fp6", 256, 256, 256, 512)
    # fewer CUs: the same shape has enough tiles; more CUs: not enough
    assert L.lpgemm_plan(L.VARIANT_I4I4, 8192, 8192, 8192, cu_count=304)["kernel"] == "fp6"
    assert L.lpgemm_plan(L.VARIANT_I4I4, 8192, 8192, 8192, cu_count=1024)["kernel"] == "fp6"   # K >= 3072
    assert L.lpgemm_plan(L.VARIANT_I4I4, 8192, 8192, 2048, cu_count=1024)["kernel"] == "tiled"
    assert L.lpgemm_plan(L.VARIANT_I4I4, 8192, 8192, 8192, cu_count=1400)["kernel"] == "tiled"
    # the FP6 path needs the fast-path conditions (K % 32, 16-byte alignment)
    assert L.lpgemm_plan(L.VARIANT_I4I4, 8192, 8192, 8194)["kernel"] == "general"
    assert L.lpgemm_plan(L.VARIANT_I4I4, 8192, 8192, 8192, B=P + 8)["kernel"] == "general"
    try:
        L.lpgemm_set_kernel_override(L.KERNEL_FP6)
        assert L.lpgemm_plan(L.VARIANT_I4I4, 1, 1, 32)["kernel"] == "fp6"
        assert L.lpgemm_plan(L.VARIANT_I4I4, 300, 5000, 64)["workgroups"] == 40
        for args in [(L.VARIANT_W4A8, 64, 64, 64), (L.VARIANT_I4I4, 64, 64, 66)]:
            with pytest.raises(L.LpgemmError) as e:
                L.lpgemm_plan(*args)
            assert e.value.status == L.ERR_UNSUPPORTED
    finally:
        L.lpgemm_set_kernel_override(L.KERNEL_AUTO)


def test_tile_size_follows_the_number_of_tiles():
    L.lpgemm_set_kernel_override(L.KERNEL_TILED)
    try:
        assert L.lpgemm_plan(L.VARIANT_I4I4, 8192, 8192, 8192)["tile_m"] == 256
    finally:
        L.lpgemm_set_kernel_override(L.KERNEL_AUTO)
    assert L.lpgemm_plan(L.VARIANT_W4A8, 4096, 4096, 4096)["tile_m"] == 256
    assert L.lpgemm_plan(L.VARIANT_I4I4, 3000, 5120, 6144)["tile_m"] == 256  # 240 tiles
    assert L.lpgemm_plan(L.VARIANT_I4I4, 2048, 2048, 2048)["tile_m"] == 128  # 256 tiles of 128
    assert L.lpgemm_plan(L.VARIANT_I4I4, 1024, 1024, 1024)["tile_m"] == 64   # 64 tiles of 128: too few
    assert L.lpgemm_plan(L.VARIANT_W4A8, 300, 260, 1056)["tile_m"] == 64
    assert L.lpgemm_plan(L.VARIANT_I4I4, 3000, 5120, 6144, cu_count=512)["tile_m"] == 128
    # 128-tiles only when they fill every compute unit; else 64-tiles, two per unit
    assert L.lpgemm_plan(L.VARIANT_I4I4, 256, 8192, 8192)["tile_m"] == 64     # 128 tiles of 128
    assert L.lpgemm_plan(L.VARIANT_W4A8, 1536, 1536, 8192)["tile_m"] == 64    # 144 tiles of 128
    assert L.lpgemm_plan(L.VARIANT_W4A8, 512, 8192, 8192)["tile_m"] == 128    # 256 tiles of 128


def test_small_m_reads_b_once_without_large_tiles_or_fp6():
    def tile(variant, M, N, K):
        p = L.lpgemm_plan(variant, M, N, K)
        return p["kernel"], p["tile_m"]
    # up to 64 rows: 128-tiles only when they fill every compute unit
    assert tile(L.VARIANT_W4A8, 32, 28672, 8192) == ("tiled", 64)    # 224 128-tiles
    assert tile(L.VARIANT_I4I4, 64, 28672, 8192) == ("tiled", 64)
    assert tile(L.VARIANT_W4A8, 64, 65536, 4096) == ("tiled", 128)   # 512 128-tiles
    assert tile(L.VARIANT_I4I4, 64, 65536, 8192) == ("tiled", 128)   # not the FP6 path
    # 65..128 rows: 128-tiles when they cover half of the compute units, never 256
    assert tile(L.VARIANT_W4A8, 100, 28672, 8192) == ("tiled", 128)
    assert tile(L.VARIANT_W4A8, 128, 65536, 4096) == ("tiled", 128)
    assert tile(L.VARIANT_I4I4, 128, 65536, 8192) == ("tiled", 128)
    assert tile(L.VARIANT_W4A8, 96, 4096, 4096) == ("tiled", 64)
    # from 129 rows the earlier rules apply again
    assert tile(L.VARIANT_I4I4, 129, 65536, 8192) == ("fp6", 256)
    assert tile(L.VARIANT_W4A8, 256, 65536, 4096) == ("tiled", 256)


def test_unaligned_pointers_take_the_general_kernel():
    assert L.lpgemm_plan(L.VARIANT_I4I4, 256, 256, 256, A=P + 1)["kernel"] == "general"
    assert L.lpgemm_plan(L.VARIANT_W4A8, 8, 256, 256, C=P + 4)["kernel"] == "general"


def test_forced_kernel_that_cannot_run_is_unsupported():
    try:
        L.lpgemm_set_kernel_override(L.KERNEL_SKINNY)
        with pytest.raises(L.LpgemmError) as e:
            L.lpgemm_plan(L.VARIANT_I4I4, 65, 256, 256)   # M above 64
        assert e.value.status == L.ERR_UNSUPPORTED
        assert L.lpgemm_plan(L.VARIANT_W4A8, 8, 256, 256)["kernel"] == "skinny"
        assert L.lpgemm_plan(L.VARIANT_I4I4, 8, 256, 256)["kernel"] == "skinny"
        L.lpgemm_set_kernel_override(L.KERNEL_TILED)
        with pytest.raises(L.LpgemmError):
            L.lpgemm_plan(L.VARIANT_W4A8, 8, 256, 34)
        L.lpgemm_set_kernel_override(L.KERNEL_GENERAL)
        assert L.lpgemm_plan(L.VARIANT_W4A8, 4096, 4096, 4096)["kernel"] == "general"
        L.lpgemm_set_kernel_override(L.KERNEL_TILED_256)
        p = L.lpgemm_plan(L.VARIANT_I4I4, 100, 100, 64)
        assert (p["kernel"], p["tile_m"], p["workgroups"]) == ("tiled", 256, 1)
        L.lpgemm_set_kernel_override(L.KERNEL_TILED_128)
        p = L.lpgemm_plan(L.VARIANT_I4I4, 8192, 8192, 8192)
        assert (p["kernel"], p["tile_m"], p["workgroups"]) == ("tiled", 128, 4096)
        L.lpgemm_set_kernel_override(L.KERNEL_TILED_64)
        p = L.lpgemm_plan(L.VARIANT_W4A8, 4096, 4096, 4096)
        assert (p["kernel"], p["tile_m"], p["workgroups"]) == ("tiled", 64, 4096)
    finally:
        L.lpgemm_set_kernel_override(L.KERNEL_AUTO)


def test_plan_grid_covers_the_output():
    for variant, M, N, K in [(L.VARIANT_I4I4, 3000, 5120, 6144), (L.VARIANT_I4I4, 1024, 1000, 64)]:
        p = L.lpgemm_plan(variant, M, N, K)
        tiles = -(-M // p["tile_m"]) * -(-N // p["tile_n"])
        assert p["workgroups"] == tiles, p
    # 256 x 256 tiles: one persistent workgroup per compute unit loops over tiles
    p = L.lpgemm_plan(L.VARIANT_I4I4, 8192, 8192, 8192)
    assert (p["tile_m"], p["workgroups"]) == (256, 256)
    assert L.lpgemm_plan(L.VARIANT_I4I4, 8192, 8192, 8192, cu_count=304)["workgroups"] == 304
    # the narrow-M kernel: one workgroup per compute unit walks the 16-row strips
    p = L.lpgemm_plan(L.VARIANT_W4A8, 16, 28672, 8192)
    assert (p["workgroups"], p["tile_n"], p["k_split"]) == (256, 16, 16)
    assert L.lpgemm_plan(L.VARIANT_W4A8, 1, 1000, 96)["workgroups"] == 63
    # capped at 256 workgroups (prefetch offsets past the end stay within 32 bits)
    assert L.lpgemm_plan(L.VARIANT_W4A8, 16, 28672, 8192, cu_count=304)["workgroups"] == 256


def test_narrow_m_limits():
    assert L.lpgemm_plan(L.VARIANT_W4A8, 16, 4096, 8192)["kernel"] == "skinny"
    assert L.lpgemm_plan(L.VARIANT_W4A8, 16, 4096, 8192)["k_chunks"] == 1
    assert L.lpgemm_plan(L.VARIANT_W4A8, 17, 28672, 4096)["kernel"] == "tiled"  # M above 16, wide N
    # N * K / 2 must stay below 2^31 (32-bit buffer offsets)
    assert L.lpgemm_plan(L.VARIANT_W4A8, 16, 65536, 65536)["kernel"] == "tiled"


def test_narrow_m_row_groups_when_forced():
    # 17..64 rows: ceil(M / 16) groups of workgroups, each set a multiple of 8
    L.lpgemm_set_kernel_override(L.KERNEL_SKINNY)
    try:
        def plan(M, N, K):
            p = L.lpgemm_plan(L.VARIANT_W4A8, M, N, K)
            return p["kernel"], p["k_chunks"], p["workgroups"]
        assert plan(32, 28672, 8192) == ("skinny", 1, 256)      # 2 groups x 128
        assert plan(48, 28672, 8192) == ("skinny", 1, 240)      # 3 groups x 80
        assert plan(64, 28672, 8192) == ("skinny", 1, 256)      # 4 groups x 64
        assert plan(64, 8192, 28672) == ("skinny", 4, 256)      # 4 groups x 4 ranges x 16
        assert plan(20, 100, 512) == ("skinny", 1, 14)          # 2 groups x 7 strips
    finally:
        L.lpgemm_set_kernel_override(L.KERNEL_AUTO)


def test_narrow_m_row_groups_automatic_choice():
    def kern(M, N, K, v=L.VARIANT_W4A8):
        return L.lpgemm_plan(v, M, N, K)["kernel"]
    assert kern(32, 4096, 4096) == "skinny"                       # 64 64-tiles < 256 CUs
    assert kern(64, 14336, 4096, L.VARIANT_I4I4) == "skinny"      # 224 64-tiles
    assert kern(32, 8192, 28672) == "skinny"                      # K in 4 ranges
    assert kern(32, 28672, 8192) == "tiled"                       # 448 64-tiles, one range
    assert kern(48, 16384, 8192, L.VARIANT_I4I4) == "tiled"       # 256 64-tiles
    assert kern(65, 4096, 4096) == "tiled"                        # above 64 rows


def test_tiled_split_k_plan():
    # automatic 64-tiles fewer than two per compute unit, K >= 12288: S = 35
    # sqrt(K / (M N)) ranges (at least 2, multiples of 256, at least 1024 k, at
    # most two workgroups per compute unit), each into its own workspace slice
    def plan(v, M, N, K):
        p = L.lpgemm_plan(v, M, N, K)
        return p["kernel"], p["tile_m"], p["k_chunks"], p["workgroups"]
    assert plan(L.VARIANT_W4A8, 128, 8192, 28672) == ("tiled", 64, 2, 512)
    assert plan(L.VARIANT_I4I4, 96, 4096, 14336) == ("tiled", 64, 4, 512)
    assert plan(L.VARIANT_W4A8, 128, 2048, 65536) == ("tiled", 64, 8, 512)
    assert plan(L.VARIANT_W4A8, 300, 300, 32768) == ("tiled", 64, 19, 475)
    assert plan(L.VARIANT_I4I4, 200, 100, 131040) == ("tiled", 64, 64, 512)
    # K below 12288, or enough tiles: one range
    assert plan(L.VARIANT_I4I4, 130, 1000, 8192) == ("tiled", 64, 1, 48)
    assert plan(L.VARIANT_I4I4, 1024, 1024, 4096) == ("tiled", 64, 1, 256)
    assert plan(L.VARIANT_I4I4, 200, 8192, 8192) == ("tiled", 64, 1, 512)
    assert plan(L.VARIANT_W4A8, 64, 28672, 8192) == ("tiled", 64, 1, 448)
    # automatic 128-tiles split only below two thirds of the compute units
    assert plan(L.VARIANT_W4A8, 128, 16384, 28672) == ("tiled", 128, 4, 512)
    assert plan(L.VARIANT_I4I4, 96, 20000, 16384) == ("tiled", 128, 3, 471)
    assert plan(L.VARIANT_I4I4, 100, 28672, 14336) == ("tiled", 128, 1, 224)
    assert plan(L.VARIANT_W4A8, 2048, 2048, 16384) == ("tiled", 128, 1, 256)
    # a forced tile size never splits
    L.lpgemm_set_kernel_override(L.KERNEL_TILED_64)
    try:
        assert plan(L.VARIANT_W4A8, 128, 2048, 65536) == ("tiled", 64, 1, 64)
    finally:
        L.lpgemm_set_kernel_override(L.KERNEL_AUTO)


def test_narrow_m_takes_both_formats():
    for v in (L.VARIANT_W4A8, L.VARIANT_I4I4):
        p = L.lpgemm_plan(v, 16, 28672, 8192)
        assert (p["kernel"], p["workgroups"], p["k_chunks"]) == ("skinny", 256, 1)
        assert L.lpgemm_plan(v, 1, 8192, 28672)["k_chunks"] == 4
        assert L.lpgemm_plan(v, 17, 28672, 8192)["kernel"] == "tiled"   # 448 64-tiles


def test_narrow_m_split_k_plan():
    # K above 8192: equal ranges of at most 8192 (multiples of 256), one group of
    # workgroups per range, the compute units shared between the groups
    def plan(M, N, K, **kw):
        p = L.lpgemm_plan(L.VARIANT_W4A8, M, N, K, **kw)
        return p["kernel"], p["k_chunks"], p["workgroups"]
    assert plan(16, 4096, 8224) == ("skinny", 2, 256)       # 2 ranges x min(256 strips, 128)
    assert plan(16, 8192, 28672) == ("skinny", 4, 256)      # 4 x 7168: 4 x 64 workgroups
    assert plan(1, 2048, 65536) == ("skinny", 8, 256)       # 128 strips, 32 workgroups per range
    assert plan(16, 64, 131040) == ("skinny", 16, 64)       # 4 strips: 16 ranges x 4, added into C
    assert plan(16, 100, 16384) == ("skinny", 2, 14)        # 7 strips per range
    assert plan(16, 8192, 28672, cu_count=304) == ("skinny", 4, 256)  # at most 256 workgroups


def test_ceiling_probe_library_loads_and_checks_arguments():
    # measurement support for bench.py: its own library, outside the GEMM's C ABI
    probe = ctypes.CDLL(os.path.join(ROOT, "precision_integer_gemm_amd", "_ceiling.so"))
    probe.ceiling_probe_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_void_p]
    probe.ceiling_probe_work.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    probe.ceiling_probe_work.restype = ctypes.c_double
    probe.ceiling_probe_out_floats.argtypes = [ctypes.c_int, ctypes.c_int]
    probe.ceiling_probe_out_floats.restype = ctypes.c_int64
    # 4 waves x 8 chains x one 32x32x64 MFMA (2 * 65536 ops) per iteration and workgroup
    assert probe.ceiling_probe_work(0, 2, 3) == 2 * 3 * 4 * 8 * 2 * 32 * 32 * 64
    assert probe.ceiling_probe_work(3, 1, 1) == 8 * 6 * 1536
    assert probe.ceiling_probe_out_floats(0, 10) == 2560
    assert probe.ceiling_probe_out_floats(4, 10) == 5120
    # rejected before any HIP call: unknown kind, empty grid, no or short output
    assert probe.ceiling_probe_run(5, 1, 1, 16, 1 << 20, None) == -1
    assert probe.ceiling_probe_run(0, 0, 1, 16, 1 << 20, None) == -1
    assert probe.ceiling_probe_run(0, 1, 1, None, 1 << 20, None) == -1
    assert probe.ceiling_probe_run(0, 4, 1, 16, 1023, None) == -1


def test_stream_probe_checks_arguments():
    # the HBM streaming-pass probe rejects bad arguments before any HIP call
    probe = ctypes.CDLL(os.path.join(ROOT, "precision_integer_gemm_amd", "_ceiling.so"))
    probe.ceiling_probe_stream_sweep.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                                 ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                                 ctypes.c_void_p]
    ok = dict(buf=256, nbytes=1 << 20, mode=0, blocks=4, threads=256, inflight=4, policy=2,
              out=256, out_ints=1024)

    def run(**kw):
        a = {**ok, **kw}
        return probe.ceiling_probe_stream_sweep(a["buf"], a["nbytes"], a["mode"], a["blocks"],
                                                a["threads"], a["inflight"], a["policy"], a["out"],
                                                a["out_ints"], None)

    assert run(buf=None) == -1
    assert run(buf=264) == -1               # not 16-byte aligned
    assert run(nbytes=0) == -1
    assert run(nbytes=(1 << 20) + 16) == -1  # not whole 1 KB pieces
    assert run(nbytes=1 << 32) == -1        # beyond a 32-bit buffer range
    assert run(blocks=0) == -1
    assert run(threads=100) == -1           # not whole waves
    assert run(out=None) == -1
    assert run(out_ints=1023) == -1         # shorter than one int per thread
    assert run(inflight=3) == -1            # not an instantiated configuration
    assert run(policy=5) == -1
    assert run(mode=1, inflight=16, threads=1024) == -1   # 256 KB of LDS
    assert run(mode=2) == -1


# ---- caller-provided workspace --------------------------------------------------
def _fp6_ws(M, N, K):
    frag = lambda R: ((R + 31) // 32) * ((K + 63) // 64) * 1536
    return (frag(M) + 255) // 256 * 256 + frag(N)


def test_workspace_size_query():
    ws = L.lpgemm_workspace_size
    assert ws(L.VARIANT_I4I4, 8192, 8192, 8192) == _fp6_ws(8192, 8192, 8192) == 100663296
    assert ws(L.VARIANT_I4I4, 8192, 8192, 8192, scaled=True) == 100663296  # FP6 serves scaled too
    assert ws(L.VARIANT_W4A8, 4096, 4096, 4096) == 0                       # int8 256-tiles
    assert ws(L.VARIANT_W4A8, 16, 28672, 8192) == 0                        # narrow-M
    assert ws(L.VARIANT_I4I4, 3000, 5120, 6144) == _fp6_ws(3000, 5120, 6144)  # FP6 from 3/4 tile per CU
    assert ws(L.VARIANT_I4I4, 2048, 4096, 4096) == 0                       # 128 tiles: int8 tiles
    assert ws(L.VARIANT_I4I4, 0, 5, 64) == 0 and ws(L.VARIANT_I4I4, 5, 5, 0) == 0
    # long K over few tiles: one int32 M x N slice per K range (int32 result only)
    p = L.lpgemm_plan(L.VARIANT_W4A8, 128, 2048, 65536)
    assert p["k_chunks"] > 1
    assert ws(L.VARIANT_W4A8, 128, 2048, 65536) == p["workspace_bytes"] == p["k_chunks"] * 128 * 2048 * 4
    assert ws(L.VARIANT_W4A8, 128, 2048, 65536, scaled=True) == 0
    assert ws(L.VARIANT_I4I4, 8192, 8192, 8192, cu_count=2048) == 0        # too few tiles for FP6
    with pytest.raises(L.LpgemmError):
        ws(L.VARIANT_I4I4, 4, 4, 33)
    with pytest.raises(L.LpgemmError):
        ws(L.VARIANT_I4I4, 4, 4, L.MAX_K + 2)
    raw = L.lib().lpgemm_workspace_size
    n = ctypes.c_size_t(7)
    assert raw(2, 0, 4, 4, 32, 0, ctypes.byref(n)) == L.ERR_INVALID_ARG    # unknown variant
    assert raw(0, 2, 4, 4, 32, 0, ctypes.byref(n)) == L.ERR_INVALID_ARG    # scaled not 0 / 1
    assert raw(0, 0, 4, 4, 32, 0, None) == L.ERR_INVALID_ARG


def test_plan_follows_the_workspace():
    need = _fp6_ws(8192, 8192, 8192)
    plan = lambda b: L.lpgemm_plan(L.VARIANT_I4I4, 8192, 8192, 8192, workspace_bytes=b)
    assert plan(0)["kernel"] == "tiled" and plan(0)["workspace_bytes"] == 0
    assert plan(need - 1)["kernel"] == "tiled"
    assert plan(need)["kernel"] == "fp6" and plan(need)["workspace_bytes"] == need
    # K ranges cut to the slices that fit; none below two
    full = L.lpgemm_plan(L.VARIANT_W4A8, 128, 2048, 65536)
    slice_ = 128 * 2048 * 4
    assert full["k_chunks"] >= 4
    cut = L.lpgemm_plan(L.VARIANT_W4A8, 128, 2048, 65536, workspace_bytes=3 * slice_ + 5)
    assert 2 <= cut["k_chunks"] <= 3 and cut["workspace_bytes"] <= 3 * slice_
    one = L.lpgemm_plan(L.VARIANT_W4A8, 128, 2048, 65536, workspace_bytes=2 * slice_ - 1)
    assert one["k_chunks"] == 1 and one["workspace_bytes"] == 0
    # a forced FP6 kernel needs its workspace
    L.lpgemm_set_kernel_override(L.KERNEL_FP6)
    try:
        assert L.lpgemm_plan(L.VARIANT_I4I4, 300, 300, 64)["kernel"] == "fp6"
        with pytest.raises(L.LpgemmError) as e:
            L.lpgemm_plan(L.VARIANT_I4I4, 300, 300, 64, workspace_bytes=0)
        assert e.value.status == L.ERR_UNSUPPORTED
    finally:
        L.lpgemm_set_kernel_override(L.KERNEL_AUTO)


@pytest.mark.parametrize("fn", ["lpgemm_int4_int4_ws", "lpgemm_w4a8_ws"])
def test_workspace_argument_errors(fn):
    f = getattr(L.lib(), fn)
    assert f(P, P, P, 4, 4, 32, None, 1024, None) == L.ERR_INVALID_ARG     # null, bytes > 0
    assert f(P, P, P, 4, 4, 32, P + 16, 1024, None) == L.ERR_INVALID_ARG   # not 256-byte aligned
    assert f(P, P, P, 4, 4, 33, P, 1024, None) == L.ERR_INVALID_ARG        # odd K still first
    assert f(P, P, P, 4, 4, L.MAX_K + 2, P, 1024, None) == L.ERR_UNSUPPORTED
    assert f(None, None, None, 0, 4, 32, None, 0, None) == L.OK             # empty
    g = L.lib().lpgemm_int4_int4_scaled_ws
    assert g(P, P, P, P, P, L.OUT_BF16, 4, 4, 32, P + 8, 64, None) == L.ERR_INVALID_ARG
    assert g(P, P, P, P, P, 9, 4, 4, 32, None, 0, None) == L.ERR_INVALID_ARG


def test_kernel_override_is_per_thread():
    import threading
    seen = {}

    def other():
        L.lpgemm_set_kernel_override(L.KERNEL_GENERAL)
        seen["other"] = L.lpgemm_plan(L.VARIANT_W4A8, 4096, 4096, 4096)["kernel"]

    L.lpgemm_set_kernel_override(L.KERNEL_AUTO)
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["other"] == "general"
    assert L.lpgemm_plan(L.VARIANT_W4A8, 4096, 4096, 4096)["kernel"] == "tiled"


def test_fp8_input_codes_are_finite_and_seeded():
    from precision_integer_gemm_amd.inputs import fp8_codes
    a = fp8_codes(5, 0, 64, 512, "e4m3")
    assert not ((a & 0x7F) == 0x7F).any() and a.shape == (64, 512)
    b = fp8_codes(5, 0, 64, 512, "e5m2")
    assert not ((b & 0x7C) == 0x7C).any()
    assert np.array_equal(fp8_codes(5, 0, 64, 512), a)            # e4m3 by default
    assert not np.array_equal(fp8_codes(5, 1, 64, 512), a)        # A and B differ
    with pytest.raises(ValueError):
        fp8_codes(5, 0, 4, 4, "e3m4")


@pytest.mark.parametrize("fn", ["lpgemm_int4_int4_blockscaled", "lpgemm_w4a8_blockscaled"])
def test_blockscaled_argument_errors(fn):
    # every rejection happens before any HIP call
    f = getattr(L.lib(), fn)
    for g in (0, 16, 48, 100, 1 << 31, -32):
        assert f(P, P, P, P, g, P, L.OUT_F32, 4, 4, 64, None) == L.ERR_INVALID_ARG, g
    assert f(P, P, P, P, 32, P, L.OUT_FP8_E4M3, 4, 4, 64, None) == L.ERR_INVALID_ARG   # fp8 out
    assert f(P, P, P, P, 32, P, 9, 4, 4, 64, None) == L.ERR_INVALID_ARG                # unknown out
    assert f(P, P, P, P, 32, P, L.OUT_F32, 4, 4, 63, None) == L.ERR_INVALID_ARG        # odd K
    assert f(P, P, P, P, 32, P, L.OUT_F32, -1, 4, 64, None) == L.ERR_INVALID_ARG       # negative M
    assert f(P, P, None, P, 32, P, L.OUT_F32, 4, 4, 64, None) == L.ERR_INVALID_ARG     # null SFA
    assert f(P, P, P, None, 32, P, L.OUT_F32, 4, 4, 64, None) == L.ERR_INVALID_ARG     # null SFB
    assert f(P, P, P + 2, P, 32, P, L.OUT_F32, 4, 4, 64, None) == L.ERR_INVALID_ARG    # misaligned SFA
    assert f(P, P, P, P, 32, P + 2, L.OUT_F32, 4, 4, 64, None) == L.ERR_INVALID_ARG    # misaligned fp32 D
    assert f(P, P, P, P, 32, P + 1, L.OUT_BF16, 4, 4, 64, None) == L.ERR_INVALID_ARG   # misaligned bf16 D
    assert f(P, P, P, P, 32, None, L.OUT_F32, 4, 4, 64, None) == L.ERR_INVALID_ARG     # null D
    assert f(P, P, P, P, 32, P, L.OUT_F32, 4, 4, L.MAX_K + 2, None) == L.ERR_UNSUPPORTED
    assert f(None, None, None, None, 32, None, L.OUT_F32, 0, 4, 64, None) == L.OK       # empty
    L.lpgemm_set_kernel_override(L.KERNEL_SKINNY)
    try:
        assert f(P, P, P, P, 32, P, L.OUT_F32, 4, 4, 64, None) == L.ERR_UNSUPPORTED
    finally:
        L.lpgemm_set_kernel_override(L.KERNEL_AUTO)


@pytest.mark.parametrize("fn,own", [("lpgemm_fp8_e4m3", L.OUT_FP8_E4M3), ("lpgemm_fp8_e5m2", L.OUT_FP8_E5M2)])
def test_fp8_argument_errors(fn, own):
    f = getattr(L.lib(), fn)
    other = L.OUT_FP8_E5M2 if own == L.OUT_FP8_E4M3 else L.OUT_FP8_E4M3
    assert f(P, P, P, other, 4, 4, 16, None) == L.ERR_INVALID_ARG     # the other format's output
    assert f(P, P, P, L.OUT_BF16, 4, 4, 16, None) == L.ERR_INVALID_ARG
    assert f(P, P, P, L.OUT_F32, -1, 4, 16, None) == L.ERR_INVALID_ARG
    assert f(P, P, None, own, 4, 4, 16, None) == L.ERR_INVALID_ARG
    assert f(P, P, P, L.OUT_F32, 4, 4, L.MAX_K + 1, None) == L.ERR_UNSUPPORTED
    assert f(None, None, None, L.OUT_F32, 0, 4, 16, None) == L.OK


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    a = torch.zeros((4, 16), dtype=torch.uint8)
    s = torch.ones((4, 1), dtype=torch.float32)
    with pytest.raises(ValueError):
        L.lpgemm_int4_int4_blockscaled(a, a, s, s, 32)
    with pytest.raises(ValueError):
        L.lpgemm_fp8_e5m2(a, a)
