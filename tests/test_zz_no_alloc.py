"""GPU test of the allocation-free entry point mmac_gemm_dense_static.

It must give exactly the bits of mmac_gemm_dense_ws with a caller-allocated
workspace (same kernels, same split-K plan), on two calls in a row that both
split K, the second with a smaller product, for bf16, int8 and fp8; and it
must pass through products that do not split (large outputs, the skinny
path).  Called through the C ABI with raw pointers.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import sparse_matrix_multiply_amd as mm
import workloads as W
from gpu_helpers import dev, to_dev_bits

pytestmark = pytest.mark.gpu


def operands(t, M, N, K, seed):
    g = np.random.default_rng(seed)
    if t == oracle.I8:
        A = g.integers(-128, 128, size=(M, K)).astype(np.int8)
        B = g.integers(-128, 128, size=(N, K)).astype(np.int8)
        C = torch.from_numpy(g.integers(-1000, 1001, size=(M, N)).astype(np.int32)).to(dev())
        return to_dev_bits(A, t), to_dev_bits(B, t), C, 1, 3
    tb = oracle.E5M2 if t == oracle.E4M3 else t
    A = W.to_bits(g.standard_normal((M, K)) / np.sqrt(K), t)
    B = W.to_bits(g.standard_normal((N, K)), tb)
    C = torch.from_numpy(g.standard_normal((M, N)).astype(np.float32)).to(dev())
    return to_dev_bits(A, t), to_dev_bits(B, tb), C, 1.25, -0.5


def static_call(t, A, B, C, alpha, beta, out_dtype):
    """mmac_gemm_dense_static through the C ABI; returns D."""
    M, K = A.shape
    N = B.shape[0]
    tb = oracle.E5M2 if t == oracle.E4M3 else t
    D = torch.full((M, N), -1, dtype=out_dtype, device=dev())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = mm.lib().mmac_gemm_dense_static(t, tb, M, N, K, float(alpha), ctypes.c_void_p(A.data_ptr()), A.stride(0),
                                         ctypes.c_void_p(B.data_ptr()), B.stride(0), float(beta),
                                         ctypes.c_void_p(C.data_ptr()), C.stride(0), ctypes.c_void_p(D.data_ptr()),
                                         D.stride(0), None, stream)
    assert st == mm.OK, mm.string(st)
    return D


def ws_call(t, A, B, C, alpha, beta, out_dtype):
    """The existing entry point, mmac_gemm_dense_ws, with a workspace the caller allocates."""
    M, K = A.shape
    N = B.shape[0]
    tb = oracle.E5M2 if t == oracle.E4M3 else t
    D = torch.full((M, N), -1, dtype=out_dtype, device=dev())
    ws = mm.workspace(t, M, N, K, device=dev())
    mm.gemm_dense(A, B, D, alpha, beta, C, a_type=t, b_type=tb, workspace=ws)
    return D


@pytest.mark.parametrize("t", [oracle.BF16, oracle.I8, oracle.E4M3])
def test_static_scratch_matches_workspace_call(t):
    out_dtype = torch.int32 if t == oracle.I8 else torch.float32
    for k, (M, N, K) in enumerate(((512, 512, 32768), (256, 256, 16384))):   # both split K; the second smaller
        assert mm.workspace_bytes(t, M, N, K) > 0
        A, B, C, alpha, beta = operands(t, M, N, K, 100 * t + k)
        Ds = static_call(t, A, B, C, alpha, beta, out_dtype)
        Dw = ws_call(t, A, B, C, alpha, beta, out_dtype)
        torch.cuda.synchronize()
        assert torch.equal(Ds.view(torch.int32), Dw.view(torch.int32)), f"call {k}: {M}x{N}x{K}"


@pytest.mark.parametrize("M,N,K", [(2048, 2048, 1024), (16, 1024, 2048)])
def test_static_scratch_without_a_split(M, N, K):
    """Products that do not split (every compute unit busy; the skinny path) use no scratch."""
    t = oracle.BF16
    assert mm.workspace_bytes(t, M, N, K) == 0
    A, B, C, alpha, beta = operands(t, M, N, K, 7)
    Ds = static_call(t, A, B, C, alpha, beta, torch.float32)
    Dw = ws_call(t, A, B, C, alpha, beta, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(Ds.view(torch.int32), Dw.view(torch.int32))
