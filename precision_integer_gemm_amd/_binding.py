"""ctypes binding of the lpgemm C-ABI (include/lpgemm.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, then their device pointers and the current HIP stream are handed
to the library.  Every step of the computation runs in the HIP kernels; there
is no fallback of any kind, and a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lpgemm.so")

# lpgemm_status
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_SCRATCH_LIMIT = 0, 1, 2, 3, 4
# lpgemm_kernel
KERNEL_AUTO, KERNEL_GENERAL, KERNEL_TILED, KERNEL_SKINNY = 0, 1, 2, 3
KERNEL_TILED_128, KERNEL_TILED_256, KERNEL_TILED_64, KERNEL_FP6 = 4, 5, 6, 7
KERNEL_NAMES = {KERNEL_AUTO: "auto", KERNEL_GENERAL: "general", KERNEL_TILED: "tiled",
                KERNEL_SKINNY: "skinny", KERNEL_FP6: "fp6"}
# lpgemm_variant
VARIANT_I4I4, VARIANT_W4A8 = 0, 1
# lpgemm_out_dtype
OUT_F32, OUT_BF16, OUT_F16, OUT_FP8_E4M3, OUT_FP8_E5M2 = 0, 1, 2, 3, 4
MAX_K = 131070

EXPORTS = ("lpgemm_int4_int4", "lpgemm_w4a8", "lpgemm_int4_int4_ws", "lpgemm_w4a8_ws",
           "lpgemm_int4_int4_noalloc",
           "lpgemm_workspace_size", "lpgemm_int4_int4_scaled", "lpgemm_w4a8_scaled",
           "lpgemm_int4_int4_scaled_ws", "lpgemm_int4_int4_blockscaled", "lpgemm_w4a8_blockscaled",
           "lpgemm_fp8_e4m3", "lpgemm_fp8_e5m2", "lpgemm_pack_int4",
           "lpgemm_unpack_int4", "lpgemm_status_string", "lpgemm_plan",
           "lpgemm_set_kernel_override")
SIZE_MAX = 2 ** 64 - 1
STATIC_SCRATCH_BYTES = 128 << 20  # LPGEMM_STATIC_SCRATCH_BYTES
WORKSPACE_ALIGN = 256


class LpgemmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lpgemm_status_string(status)} (status {status})")


class PlanInfo(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("tile_m", ctypes.c_int32),
                ("tile_n", ctypes.c_int32), ("k_split", ctypes.c_int32),
                ("workgroups", ctypes.c_int64), ("threads", ctypes.c_int32),
                ("k_chunks", ctypes.c_int32), ("workspace_bytes", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {"kernel": KERNEL_NAMES.get(self.kernel, self.kernel), "tile_m": self.tile_m,
                "tile_n": self.tile_n, "k_split": self.k_split,
                "workgroups": self.workgroups, "threads": self.threads,
                "k_chunks": self.k_chunks, "workspace_bytes": self.workspace_bytes}


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"the HIP library {LIB_PATH} is not built; run "
                          "`python -m precision_integer_gemm_amd.build` (or __graft_entry__.build())")
    # PyTorch brings its own HIP runtime: load it first, so that the library
    # binds to the same runtime as the streams and device pointers PyTorch
    # hands over (a second runtime loaded ahead of it leaves PyTorch without
    # a device).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    sz = ctypes.c_size_t
    for name in ("lpgemm_int4_int4", "lpgemm_w4a8", "lpgemm_int4_int4_noalloc"):
        f = getattr(L, name)
        f.argtypes = [p, p, p, i64, i64, i64, p]
        f.restype = ctypes.c_int
    for name in ("lpgemm_int4_int4_ws", "lpgemm_w4a8_ws"):
        f = getattr(L, name)
        f.argtypes = [p, p, p, i64, i64, i64, p, sz, p]
        f.restype = ctypes.c_int
    L.lpgemm_workspace_size.argtypes = [ctypes.c_int, i32, i64, i64, i64, i32, ctypes.POINTER(sz)]
    L.lpgemm_workspace_size.restype = ctypes.c_int
    for name in ("lpgemm_int4_int4_scaled", "lpgemm_w4a8_scaled"):
        f = getattr(L, name)
        f.argtypes = [p, p, p, p, p, ctypes.c_int, i64, i64, i64, p]
        f.restype = ctypes.c_int
    L.lpgemm_int4_int4_scaled_ws.argtypes = [p, p, p, p, p, ctypes.c_int, i64, i64, i64, p, sz, p]
    L.lpgemm_int4_int4_scaled_ws.restype = ctypes.c_int
    for name in ("lpgemm_int4_int4_blockscaled", "lpgemm_w4a8_blockscaled"):
        f = getattr(L, name)
        f.argtypes = [p, p, p, p, i64, p, ctypes.c_int, i64, i64, i64, p]
        f.restype = ctypes.c_int
    for name in ("lpgemm_fp8_e4m3", "lpgemm_fp8_e5m2"):
        getattr(L, name).argtypes = [p, p, p, ctypes.c_int, i64, i64, i64, p]
        getattr(L, name).restype = ctypes.c_int
    for name in ("lpgemm_pack_int4", "lpgemm_unpack_int4"):
        f = getattr(L, name)
        f.argtypes = [p, p, i64, i64, p]
        f.restype = ctypes.c_int
    L.lpgemm_status_string.argtypes = [ctypes.c_int]
    L.lpgemm_status_string.restype = ctypes.c_char_p
    L.lpgemm_plan.argtypes = [ctypes.c_int, p, p, p, i64, i64, i64, sz, i32, ctypes.POINTER(PlanInfo)]
    L.lpgemm_plan.restype = ctypes.c_int
    L.lpgemm_set_kernel_override.argtypes = [ctypes.c_int]
    L.lpgemm_set_kernel_override.restype = ctypes.c_int
    _lib = L
    return L


def lpgemm_status_string(status: int) -> str:
    return lib().lpgemm_status_string(int(status)).decode()


def _raise(status: int, what: str) -> None:
    if status != OK:
        raise LpgemmError(status, what)


def lpgemm_plan(variant: int, M: int, N: int, K: int, A: int = 256, B: int = 256, C: int = 256,
                cu_count: int = 0, workspace_bytes: int | None = None) -> dict:
    """Kernel and launch shape a call would use (host only; pointers are plain
    integers, inspected only for alignment).  workspace_bytes None: a call
    given all the workspace it can use; 0: a call without workspace."""
    info = PlanInfo()
    ws = SIZE_MAX if workspace_bytes is None else int(workspace_bytes)
    _raise(lib().lpgemm_plan(variant, A, B, C, M, N, K, ws, cu_count, ctypes.byref(info)),
           "lpgemm_plan")
    return info.as_dict()


def lpgemm_workspace_size(variant: int, M: int, N: int, K: int, scaled: bool = False,
                          cu_count: int = 0) -> int:
    """Bytes of workspace a "_ws" call with these sizes can use (host only)."""
    n = ctypes.c_size_t(0)
    _raise(lib().lpgemm_workspace_size(variant, int(bool(scaled)), M, N, K, cu_count,
                                       ctypes.byref(n)), "lpgemm_workspace_size")
    return int(n.value)


def lpgemm_set_kernel_override(kernel: int) -> None:
    _raise(lib().lpgemm_set_kernel_override(int(kernel)), "lpgemm_set_kernel_override")


# ---- tensor-level calls ------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream_handle(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check_dev(t, name: str, dtypes):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(workspace, variant, M, N, K, scaled, device):
    """(pointer, bytes) of the workspace for a tensor-level call: "auto"
    allocates what the call can use through PyTorch's allocator (none when the
    call needs none), None passes none, a uint8 tensor on the device is used
    as given (aligned to 256 bytes inside it)."""
    torch = _torch()
    if workspace is None:
        return None, 0, None
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", None or a uint8 tensor')
        n = lpgemm_workspace_size(variant, M, N, K, scaled=scaled)
        if n == 0:
            return None, 0, None
        workspace = torch.empty(n + WORKSPACE_ALIGN, dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8 or \
            workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous uint8 tensor on a GPU device")
    base = workspace.data_ptr()
    skip = (-base) % WORKSPACE_ALIGN
    n = max(0, workspace.numel() - skip)
    return (base + skip if n else None), n, workspace


def _out(out, M, N, device):
    torch = _torch()
    if out is None:
        return torch.empty((M, N), dtype=torch.int32, device=device)
    _check_dev(out, "out", (torch.int32,))
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must have shape ({M}, {N}), got {tuple(out.shape)}")
    return out


def lpgemm_int4_int4(A_packed, B_packed, *, out=None, workspace="auto", stream=None):
    """C[M,N] int32 = A . B^T with both operands packed int4 ([M,K/2], [N,K/2]).
    workspace: "auto" (allocated through PyTorch when the call can use one),
    None (the entry point without workspace) or a uint8 device tensor."""
    torch = _torch()
    _check_dev(A_packed, "A_packed", (torch.int8, torch.uint8))
    _check_dev(B_packed, "B_packed", (torch.int8, torch.uint8))
    M, half = A_packed.shape
    N, half_b = B_packed.shape
    if half != half_b:
        raise ValueError(f"packed K mismatch: A has {half} bytes per row, B {half_b}")
    C = _out(out, M, N, A_packed.device)
    ws, nws, _keep = _workspace(workspace, VARIANT_I4I4, M, N, 2 * half, False, A_packed.device)
    if nws:
        _raise(lib().lpgemm_int4_int4_ws(A_packed.data_ptr(), B_packed.data_ptr(), C.data_ptr(),
                                         M, N, 2 * half, ws, nws, _stream_handle(stream)),
               "lpgemm_int4_int4_ws")
    else:
        _raise(lib().lpgemm_int4_int4(A_packed.data_ptr(), B_packed.data_ptr(), C.data_ptr(),
                                      M, N, 2 * half, _stream_handle(stream)), "lpgemm_int4_int4")
    return C


def lpgemm_w4a8(A, B_packed, *, out=None, workspace="auto", stream=None):
    """C[M,N] int32 = A . B^T with A int8 [M,K] and B packed int4 [N,K/2];
    workspace as for lpgemm_int4_int4."""
    torch = _torch()
    _check_dev(A, "A", (torch.int8,))
    _check_dev(B_packed, "B_packed", (torch.uint8, torch.int8))
    M, K = A.shape
    N, half = B_packed.shape
    if K != 2 * half:
        raise ValueError(f"K mismatch: A has K={K}, B_packed holds {2 * half}")
    C = _out(out, M, N, A.device)
    ws, nws, _keep = _workspace(workspace, VARIANT_W4A8, M, N, K, False, A.device)
    if nws:
        _raise(lib().lpgemm_w4a8_ws(A.data_ptr(), B_packed.data_ptr(), C.data_ptr(), M, N, K,
                                    ws, nws, _stream_handle(stream)), "lpgemm_w4a8_ws")
    else:
        _raise(lib().lpgemm_w4a8(A.data_ptr(), B_packed.data_ptr(), C.data_ptr(), M, N, K,
                                 _stream_handle(stream)), "lpgemm_w4a8")
    return C


def _out_code(dtype):
    torch = _torch()
    codes = {torch.float32: OUT_F32, torch.bfloat16: OUT_BF16, torch.float16: OUT_F16}
    if dtype not in codes:
        raise TypeError(f"out dtype must be one of {list(codes)}, got {dtype}")
    return codes[dtype]


def _scaled_out(out, dtype, M, N, device):
    torch = _torch()
    if out is None:
        return torch.empty((M, N), dtype=dtype, device=device)
    _check_dev(out, "out", (dtype,))
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must have shape ({M}, {N}), got {tuple(out.shape)}")
    return out


def _check_scales(scale_a, scale_b, M, N):
    torch = _torch()
    for name, t, n in (("scale_a", scale_a, M), ("scale_b", scale_b, N)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dtype != torch.float32:
            raise TypeError(f"{name} must be a float32 tensor on a GPU device")
        if t.dim() != 1 or t.shape[0] != n or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous with shape ({n},)")


def lpgemm_int4_int4_scaled(A_packed, B_packed, scale_a, scale_b, *, dtype=None, out=None,
                            workspace="auto", stream=None):
    """D[M,N] = out(((float)C * scale_a[m]) * scale_b[n]) of the int4 x int4 product C;
    workspace as for lpgemm_int4_int4."""
    torch = _torch()
    _check_dev(A_packed, "A_packed", (torch.int8, torch.uint8))
    _check_dev(B_packed, "B_packed", (torch.int8, torch.uint8))
    M, half = A_packed.shape
    N, half_b = B_packed.shape
    if half != half_b:
        raise ValueError(f"packed K mismatch: A has {half} bytes per row, B {half_b}")
    _check_scales(scale_a, scale_b, M, N)
    dtype = dtype or (out.dtype if out is not None else torch.bfloat16)
    D = _scaled_out(out, dtype, M, N, A_packed.device)
    ws, nws, _keep = _workspace(workspace, VARIANT_I4I4, M, N, 2 * half, True, A_packed.device)
    if nws:
        _raise(lib().lpgemm_int4_int4_scaled_ws(A_packed.data_ptr(), B_packed.data_ptr(),
                                                scale_a.data_ptr(), scale_b.data_ptr(),
                                                D.data_ptr(), _out_code(dtype), M, N, 2 * half,
                                                ws, nws, _stream_handle(stream)),
               "lpgemm_int4_int4_scaled_ws")
    else:
        _raise(lib().lpgemm_int4_int4_scaled(A_packed.data_ptr(), B_packed.data_ptr(),
                                             scale_a.data_ptr(), scale_b.data_ptr(), D.data_ptr(),
                                             _out_code(dtype), M, N, 2 * half,
                                             _stream_handle(stream)),
               "lpgemm_int4_int4_scaled")
    return D


def lpgemm_w4a8_scaled(A, B_packed, scale_a, scale_b, *, dtype=None, out=None, stream=None):
    """D[M,N] = out(((float)C * scale_a[m]) * scale_b[n]) of the W4A8 product C."""
    torch = _torch()
    _check_dev(A, "A", (torch.int8,))
    _check_dev(B_packed, "B_packed", (torch.uint8, torch.int8))
    M, K = A.shape
    N, half = B_packed.shape
    if K != 2 * half:
        raise ValueError(f"K mismatch: A has K={K}, B_packed holds {2 * half}")
    _check_scales(scale_a, scale_b, M, N)
    dtype = dtype or (out.dtype if out is not None else torch.bfloat16)
    D = _scaled_out(out, dtype, M, N, A.device)
    _raise(lib().lpgemm_w4a8_scaled(A.data_ptr(), B_packed.data_ptr(), scale_a.data_ptr(),
                                    scale_b.data_ptr(), D.data_ptr(), _out_code(dtype), M, N, K,
                                    _stream_handle(stream)), "lpgemm_w4a8_scaled")
    return D


def _check_block_scales(SFA, SFB, M, N, K, g):
    torch = _torch()
    nb = -(-K // g) if g > 0 else 0
    for name, t, n in (("SFA", SFA, M), ("SFB", SFB, N)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dtype != torch.float32:
            raise TypeError(f"{name} must be a float32 tensor on a GPU device")
        if tuple(t.shape) != (n, nb) or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous with shape ({n}, {nb}) for K={K}, g={g}")


def lpgemm_int4_int4_blockscaled(A_packed, B_packed, SFA, SFB, g, *, dtype=None, out=None, stream=None):
    """D[M,N] = out(sum_j ((float)C_j * SFA[m,j]) * SFB[n,j]) over the K blocks
    of g (a power of two >= 32) of the int4 x int4 product, added in block order
    in binary32; SFA [M, ceil(K/g)], SFB [N, ceil(K/g)] float32."""
    torch = _torch()
    _check_dev(A_packed, "A_packed", (torch.int8, torch.uint8))
    _check_dev(B_packed, "B_packed", (torch.int8, torch.uint8))
    M, half = A_packed.shape
    N, half_b = B_packed.shape
    if half != half_b:
        raise ValueError(f"packed K mismatch: A has {half} bytes per row, B {half_b}")
    _check_block_scales(SFA, SFB, M, N, 2 * half, g)
    dtype = dtype or (out.dtype if out is not None else torch.bfloat16)
    D = _scaled_out(out, dtype, M, N, A_packed.device)
    _raise(lib().lpgemm_int4_int4_blockscaled(A_packed.data_ptr(), B_packed.data_ptr(), SFA.data_ptr(),
                                              SFB.data_ptr(), g, D.data_ptr(), _out_code(dtype), M, N,
                                              2 * half, _stream_handle(stream)),
           "lpgemm_int4_int4_blockscaled")
    return D


def lpgemm_w4a8_blockscaled(A, B_packed, SFA, SFB, g, *, dtype=None, out=None, stream=None):
    """lpgemm_int4_int4_blockscaled for int8 A [M, K] and packed int4 B."""
    torch = _torch()
    _check_dev(A, "A", (torch.int8,))
    _check_dev(B_packed, "B_packed", (torch.uint8, torch.int8))
    M, K = A.shape
    N, half = B_packed.shape
    if K != 2 * half:
        raise ValueError(f"K mismatch: A has K={K}, B_packed holds {2 * half}")
    _check_block_scales(SFA, SFB, M, N, K, g)
    dtype = dtype or (out.dtype if out is not None else torch.bfloat16)
    D = _scaled_out(out, dtype, M, N, A.device)
    _raise(lib().lpgemm_w4a8_blockscaled(A.data_ptr(), B_packed.data_ptr(), SFA.data_ptr(), SFB.data_ptr(),
                                         g, D.data_ptr(), _out_code(dtype), M, N, K, _stream_handle(stream)),
           "lpgemm_w4a8_blockscaled")
    return D


def _fp8_gemm(name, f8_name, own_code, A, B, dtype, out, stream):
    torch = _torch()
    f8 = getattr(torch, f8_name, None)
    ok = (torch.uint8,) + ((f8,) if f8 is not None else ())
    _check_dev(A, "A", ok)
    _check_dev(B, "B", ok)
    M, K = A.shape
    N, K_b = B.shape
    if K != K_b:
        raise ValueError(f"K mismatch: A has K={K}, B has {K_b}")
    dtype = dtype or (out.dtype if out is not None else torch.float32)
    if dtype == torch.float32:
        code = OUT_F32
    elif dtype in ok:
        code = own_code
    else:
        raise TypeError(f"dtype must be torch.float32, torch.uint8 or torch.{f8_name}")
    if out is None:
        C = torch.empty((M, N), dtype=dtype, device=A.device)
    else:
        _check_dev(out, "out", (dtype,))
        if tuple(out.shape) != (M, N):
            raise ValueError(f"out must have shape ({M}, {N}), got {tuple(out.shape)}")
        C = out
    _raise(getattr(lib(), name)(A.data_ptr(), B.data_ptr(), C.data_ptr(), code, M, N, K,
                                _stream_handle(stream)), name)
    return C


def lpgemm_fp8_e4m3(A, B, *, dtype=None, out=None, stream=None):
    """C[M,N] = A . B^T of e4m3 operands (uint8 codes or torch.float8_e4m3fn
    tensors [M,K] and [N,K]) with fp32 accumulation; C as float32 (default) or
    e4m3 codes (dtype=torch.uint8 or torch.float8_e4m3fn)."""
    return _fp8_gemm("lpgemm_fp8_e4m3", "float8_e4m3fn", OUT_FP8_E4M3, A, B, dtype, out, stream)


def lpgemm_fp8_e5m2(A, B, *, dtype=None, out=None, stream=None):
    """C[M,N] = A . B^T of e5m2 operands (uint8 codes or torch.float8_e5m2
    tensors [M,K] and [N,K]) with fp32 accumulation; C as float32 (default) or
    e5m2 codes (dtype=torch.uint8 or torch.float8_e5m2)."""
    return _fp8_gemm("lpgemm_fp8_e5m2", "float8_e5m2", OUT_FP8_E5M2, A, B, dtype, out, stream)


def lpgemm_pack_int4(logical, *, out=None, stream=None):
    """Logical int4 values held as int8 [rows, K] -> packed uint8 [rows, K/2]."""
    torch = _torch()
    _check_dev(logical, "logical", (torch.int8,))
    rows, K = logical.shape
    if K % 2:
        raise ValueError("the last dimension of a logical int4 tensor must be even")
    if out is None:
        out = torch.empty((rows, K // 2), dtype=torch.uint8, device=logical.device)
    else:
        _check_dev(out, "out", (torch.uint8, torch.int8))
        if tuple(out.shape) != (rows, K // 2):
            raise ValueError("out has the wrong shape")
    _raise(lib().lpgemm_pack_int4(logical.data_ptr(), out.data_ptr(), rows, K,
                                  _stream_handle(stream)), "lpgemm_pack_int4")
    return out


def lpgemm_unpack_int4(packed, *, out=None, stream=None):
    """Packed bytes [rows, K/2] -> logical int4 values as int8 [rows, K]."""
    torch = _torch()
    _check_dev(packed, "packed", (torch.uint8, torch.int8))
    rows, half = packed.shape
    if out is None:
        out = torch.empty((rows, 2 * half), dtype=torch.int8, device=packed.device)
    else:
        _check_dev(out, "out", (torch.int8,))
        if tuple(out.shape) != (rows, 2 * half):
            raise ValueError("out has the wrong shape")
    _raise(lib().lpgemm_unpack_int4(packed.data_ptr(), out.data_ptr(), rows, 2 * half,
                                    _stream_handle(stream)), "lpgemm_unpack_int4")
    return out
