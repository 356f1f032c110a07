"""lpgemm -- exact low-precision integer GEMM for AMD MI355X (gfx950).

    C[M,N] = A[M,K] . B[N,K]^T   (int32), A and B int4 packed two per byte
                                  (int4 x int4) or A int8 with B packed (W4A8);
    D[M,N] = out(((float)C * scale_a[m]) * scale_b[n])   (fp32, bf16 or fp16),
    and per K block of g: D = out(sum_j ((float)C_j * SFA[m,j]) * SFB[n,j]).

The computation runs in hand-written HIP kernels behind a C ABI
(include/lpgemm.h, built into _lpgemm.so); this package is the thin Python
binding with the same entry-point names.  PyTorch provides device memory and
streams only.
"""
from ._binding import (  # noqa: F401
    ERR_HIP, ERR_INVALID_ARG, ERR_SCRATCH_LIMIT, ERR_UNSUPPORTED, EXPORTS, KERNEL_AUTO, KERNEL_GENERAL,
    KERNEL_FP6, KERNEL_NAMES, KERNEL_SKINNY, KERNEL_TILED, KERNEL_TILED_128, KERNEL_TILED_256, KERNEL_TILED_64,
    LIB_PATH, MAX_K,
    OK, OUT_BF16, OUT_F16, OUT_F32, OUT_FP8_E4M3, OUT_FP8_E5M2, VARIANT_I4I4, VARIANT_W4A8, LpgemmError, lib,
    lpgemm_fp8_e4m3, lpgemm_fp8_e5m2, lpgemm_int4_int4, lpgemm_int4_int4_blockscaled, lpgemm_int4_int4_scaled, lpgemm_pack_int4, lpgemm_plan,
    lpgemm_set_kernel_override, lpgemm_status_string, lpgemm_unpack_int4, lpgemm_w4a8,
    lpgemm_w4a8_blockscaled, lpgemm_w4a8_scaled, lpgemm_workspace_size, SIZE_MAX, STATIC_SCRATCH_BYTES, WORKSPACE_ALIGN)
