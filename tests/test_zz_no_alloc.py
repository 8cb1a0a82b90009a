"""bi_gemm_splitk_noalloc, the allocation-free split-K GEMM, against
bi_gemm_splitk (the same kernels with the caller's workspace): both called
through the C ABI, two calls in a row, the second smaller than the first, so
that the second one runs over what the first left in the static scratch."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
from invariant_deterministic_amd import synth, workloads
from tests.gpu_util import check_bf16, dev_bf16, host_u16, need_gpu, say

pytestmark = pytest.mark.gpu

BI_OK, BI_ERR_WORKSPACE = 0, 4


@pytest.fixture(scope="module")
def lib():
    need_gpu()
    from invariant_deterministic_amd import binding
    L = binding.raw()
    p, i64, i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.bi_gemm_splitk_noalloc.argtypes = [p, p, p, i64, i64, i64, i64, i64, i64, i, p]
    L.bi_gemm_splitk.argtypes = [p, p, p, i64, i64, i64, i64, i64, i64, i, p, ctypes.c_size_t, p]
    L.bi_gemm_splitk_for.argtypes = [i64, i64]
    L.bi_gemm_splitk_workspace_bytes.argtypes = [i64, i64, i]
    L.bi_gemm_splitk_workspace_bytes.restype = ctypes.c_size_t
    return L


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _run_both(lib, X, Wt, M, N, K, S):
    """(noalloc output, workspace output) for the first M rows of X."""
    ya = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    yb = torch.full((M, N), -7.0, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(lib.bi_gemm_splitk_workspace_bytes(M, N, S), dtype=torch.uint8, device="cuda")
    st = lib.bi_gemm_splitk_noalloc(X.data_ptr(), Wt.data_ptr(), ya.data_ptr(), M, N, K, K, K, N, S,
                                    _stream())
    assert st == BI_OK, st
    st = lib.bi_gemm_splitk(X.data_ptr(), Wt.data_ptr(), yb.data_ptr(), M, N, K, K, K, N, S,
                            ws.data_ptr(), ws.numel(), _stream())
    assert st == BI_OK, st
    return host_u16(ya), host_u16(yb)


def test_noalloc_equals_workspace_entry_point(lib):
    """Up projection (K = 4096, N = 14336, split 4) at M = 64, then KV
    (N = 1024, split 16) at M = 5: bit for bit equal to bi_gemm_splitk, and the
    sampled rows within tolerance of the oracle."""
    c = workloads.LLAMA8B
    x = workloads.llama8b_x(4096, rows=64)
    X = dev_bf16(x)
    for si, M in ((2, 64), (1, 5)):
        K, N = c["shapes"][si]
        w = workloads.llama8b_w(si)
        Wt = dev_bf16(w)
        S = lib.bi_gemm_splitk_for(N, K)
        say(f"noalloc split-K K={K} N={N} M={M} S={S}")
        a, b = _run_both(lib, X, Wt, M, N, K, S)
        assert np.array_equal(a, b), int((a != b).sum())
        rows = np.array(sorted({0, M // 2, M - 1}))
        check_bf16(a[rows], oracle.gemm(x[rows], w), f"noalloc K={K} N={N} M={M}")


def test_noalloc_rejects_a_request_beyond_the_scratch(lib):
    """8 * 129 * 4096 fp32 partials exceed the 16 MiB scratch: the call is
    refused before anything runs, and the output is untouched."""
    K = N = 4096
    X = dev_bf16(synth.normal_bf16((129, K), 71))
    Wt = dev_bf16(synth.normal_bf16((N, K), 72, std=0.02))
    y = torch.full((129, N), 3.0, dtype=torch.bfloat16, device="cuda")
    st = lib.bi_gemm_splitk_noalloc(X.data_ptr(), Wt.data_ptr(), y.data_ptr(), 129, N, K, K, K, N, 8,
                                    _stream())
    assert st == BI_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
    a, b = _run_both(lib, X, Wt, 128, N, K, 8)     # exactly 16 MiB: accepted
    assert np.array_equal(a, b)
