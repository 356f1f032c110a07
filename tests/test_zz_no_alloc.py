"""The allocation-free entry point lpgemm_int4_int4_noalloc: the same product as
lpgemm_int4_int4_ws, with the library's static scratch as the workspace.

Its results are compared bit for bit with the workspace entry point's (each
call there with a workspace of its own) and with the oracle, on calls in a
row that use the scratch differently: the FP6 re-encoding of a large product,
a smaller forced-FP6 product over the first part of the same scratch (stale
bytes of the first call behind it), and a split-K product whose partial-sum
slices reuse it again.
"""
import sys

import numpy as np
import pytest

import oracle
import precision_integer_gemm_amd as L
from precision_integer_gemm_amd.inputs import custom_operands

SENTINEL = 0x7EADBEEF
GUARD = 1024


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_scratch_limit_and_argument_errors_on_the_host():
    f = L.lib().lpgemm_int4_int4_noalloc
    P = 4096
    # the FP6 path of 16384 x 16384 x 8192 needs 192 MiB: rejected before any launch
    need = L.lpgemm_workspace_size(L.VARIANT_I4I4, 16384, 16384, 8192)
    assert need > L.STATIC_SCRATCH_BYTES
    assert f(P, P, P, 16384, 16384, 8192, None) == L.ERR_SCRATCH_LIMIT
    assert L.lpgemm_status_string(L.ERR_SCRATCH_LIMIT).startswith("needs more scratch")
    assert L.lpgemm_workspace_size(L.VARIANT_I4I4, 8192, 8192, 8192) <= L.STATIC_SCRATCH_BYTES
    # argument errors as lpgemm_int4_int4, ahead of the scratch check
    assert f(P, P, P, 4, 4, 33, None) == L.ERR_INVALID_ARG
    assert f(P, P, None, 4, 4, 32, None) == L.ERR_INVALID_ARG
    assert f(P, P, P, -1, 4, 32, None) == L.ERR_INVALID_ARG
    assert f(P, P, P, 4, 4, L.MAX_K + 2, None) == L.ERR_UNSUPPORTED
    assert f(None, None, None, 0, 4, 32, None) == L.OK


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


def _call(torch, A, B, M, N, K, noalloc):
    dev = torch.device("cuda:0")
    a_t = torch.from_numpy(np.ascontiguousarray(A).view(np.uint8).reshape(-1)).to(dev)
    b_t = torch.from_numpy(np.ascontiguousarray(B).reshape(-1)).to(dev)
    cbuf = torch.full((M * N + 2 * GUARD,), SENTINEL, dtype=torch.int32, device=dev)
    c_t = cbuf[GUARD:GUARD + M * N]
    s = torch.cuda.current_stream().cuda_stream
    if noalloc:
        st = L.lib().lpgemm_int4_int4_noalloc(a_t.data_ptr(), b_t.data_ptr(), c_t.data_ptr(),
                                              M, N, K, s)
    else:
        nws = L.lpgemm_plan(L.VARIANT_I4I4, M, N, K)["workspace_bytes"]
        ws = torch.empty(nws + L.WORKSPACE_ALIGN, dtype=torch.uint8, device=dev)
        ptr = ws.data_ptr() + (-ws.data_ptr()) % L.WORKSPACE_ALIGN
        st = L.lib().lpgemm_int4_int4_ws(a_t.data_ptr(), b_t.data_ptr(), c_t.data_ptr(), M, N, K,
                                         ptr, nws, s)
    assert st == L.OK, L.lpgemm_status_string(st)
    torch.cuda.synchronize()
    host = cbuf.cpu().numpy()
    assert (host[:GUARD] == SENTINEL).all() and (host[GUARD + M * N:] == SENTINEL).all()
    return host[GUARD:GUARD + M * N].reshape(M, N)


# (M, N, K, forced kernel, the path that must use the scratch)
CALLS = [(4096, 4096, 8192, L.KERNEL_AUTO, "fp6"),
         (1000, 513, 4160, L.KERNEL_FP6, "fp6"),
         (200, 100, 131040, L.KERNEL_AUTO, "split")]


@pytest.mark.gpu
def test_noalloc_matches_the_workspace_entry_point_on_calls_in_a_row(torch):
    for i, (M, N, K, kernel, path) in enumerate(CALLS):
        L.lpgemm_set_kernel_override(kernel)
        plan = L.lpgemm_plan(L.VARIANT_I4I4, M, N, K)
        say(f"noalloc call {i}: {M}x{N}x{K} kernel {kernel} plan={plan}")
        assert 0 < plan["workspace_bytes"] <= L.STATIC_SCRATCH_BYTES
        assert (plan["kernel"] == "fp6") if path == "fp6" else (plan["k_chunks"] > 1)
        A, B = custom_operands("i4i4", M, N, K, seed=4000 + i)
        got = _call(torch, A, B, M, N, K, noalloc=True)
        ref = _call(torch, A, B, M, N, K, noalloc=False)
        assert np.array_equal(got, ref)
        assert np.array_equal(got, oracle.gemm_i4i4(A, B, M, N, K))
    # the first shape again after the others: the scratch holds stale data
    M, N, K, kernel, _ = CALLS[0]
    L.lpgemm_set_kernel_override(kernel)
    A, B = custom_operands("i4i4", M, N, K, seed=4000)
    assert np.array_equal(_call(torch, A, B, M, N, K, noalloc=True),
                          _call(torch, A, B, M, N, K, noalloc=False))
