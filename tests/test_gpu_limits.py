"""GPU parity at the interface's size limits.  The tiled and skinny kernels address a 256-row
(or 16-row) slab of an operand with one buffer resource and 32-bit offsets, so the library caps
row pitches at 8 MiB (2 Mi words for the 4:2 index) and a transposed operand at K rows below
2 GiB; here every operand and output sits at that cap, where a 256-row tile spans the whole
2 GiB a 32-bit offset reaches.  The compressor, under the same cap, addresses rows with 64-bit
pointers: with 600 rows at the largest pitch its last rows lie beyond 4 GiB.  Small M, N and K
keep the oracle quick; the pitches make the buffers several GiB of (zeroed) GPU memory.  One
step past the caps the calls return MMAC_ERR_UNSUPPORTED (tests/test_abi_host.py)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_matrix_multiply_amd as mm
import workloads as W
from gpu_helpers import ESIZE, assert_close, dev, dev_bits_to_host, out_tensor, tile_shape, to_dev_bits
from oracle import BF16, E4M3, E5M2, F16, I8
from test_gpu_sparse import sparse_a

pytestmark = pytest.mark.gpu

MAX_PITCH = 1 << 23          # bytes of a row
# bytes of a row of a transposed operand with K = 640 rows: the largest multiple of 16 with
# 640 rows below 2 GiB
T_K = 640
T_PITCH = ((1 << 31) - 1) // T_K // 16 * 16


def max_ld(t):
    return MAX_PITCH // ESIZE[t]


def inputs(ta, tb, M, N, K, seed):
    g = np.random.default_rng(seed)
    if ta == I8:
        A = g.integers(-128, 128, size=(M, K)).astype(np.int8)
        B = g.integers(-128, 128, size=(N, K)).astype(np.int8)
        C = g.integers(-1000, 1001, size=(M, N)).astype(np.int32)
        return A, B, C, 1, 1
    A = W.to_bits(g.standard_normal((M, K)), ta)
    B = W.to_bits(g.standard_normal((N, K)) / np.sqrt(K), tb)
    C = g.standard_normal((M, N)).astype(np.float32)
    return A, B, C, 0.5, -1.0


def check(D, Dref, S, ta, K, alpha, beta, C, what):
    if ta == I8:
        assert np.array_equal(D, Dref), what
    else:
        assert_close(D, Dref, S, ta, K, alpha, beta, C, what)


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("ta,tb", [(BF16, BF16), (I8, I8), (E4M3, E5M2)])
@pytest.mark.parametrize("shape", [None, 256])
def test_dense_at_max_row_pitch(ta, tb, shape):
    """A, B, C and D all at the largest pitch; with shape 256 a 256-row tile of A spans 2 GiB."""
    M, N, K = 300, 260, 640
    A, B, C, alpha, beta = inputs(ta, tb, M, N, K, 5 + ta)
    Ad, Bd = to_dev_bits(A, ta, max_ld(ta)), to_dev_bits(B, tb, max_ld(tb))
    D = out_tensor(M, N, ta == I8, MAX_PITCH // 4)
    Cbuf = torch.zeros((M, MAX_PITCH // 4), dtype=torch.int32 if ta == I8 else torch.float32, device=dev())
    Cbuf[:, :N] = torch.from_numpy(C).to(dev())
    Cd = Cbuf[:, :N]
    if shape is None:
        mm.gemm_dense(Ad, Bd, D, alpha, beta, Cd, a_type=ta, b_type=tb)
    else:
        with tile_shape(shape):
            mm.gemm_dense(Ad, Bd, D, alpha, beta, Cd, a_type=ta, b_type=tb)
    torch.cuda.synchronize()
    Dref, S = oracle.gemm_dense(ta, tb, A, B, alpha, beta, C)
    check(D.cpu().numpy(), Dref, S, ta, K, alpha, beta, C, f"max pitch {ta},{tb} tile {shape}")


@pytest.mark.parametrize("ta,tb", [(BF16, BF16), (I8, I8), (E4M3, E5M2)])
def test_skinny_at_max_row_pitch(ta, tb):
    M, N, K = 20, 300, 1000
    A, B, C, alpha, beta = inputs(ta, tb, M, N, K, 9 + ta)
    Ad, Bd = to_dev_bits(A, ta, max_ld(ta)), to_dev_bits(B, tb, max_ld(tb))
    D = out_tensor(M, N, ta == I8, MAX_PITCH // 4)
    Cd = torch.from_numpy(C).to(dev())
    mm.gemm_dense(Ad, Bd, D, alpha, beta, Cd, a_type=ta, b_type=tb)
    torch.cuda.synchronize()
    Dref, S = oracle.gemm_dense(ta, tb, A, B, alpha, beta, C)
    check(D.cpu().numpy(), Dref, S, ta, K, alpha, beta, C, f"skinny max pitch {ta},{tb}")


@pytest.mark.parametrize("ta,tb", [(BF16, BF16), (I8, I8), (E4M3, E5M2)])
def test_layout_at_max_transposed_span(ta, tb):
    """A given K x M and B given K x N, each K rows spanning just under 2 GiB."""
    M, N, K = 300, 260, T_K
    A, B, C, alpha, beta = inputs(ta, tb, M, N, K, 13 + ta)
    assert K * T_PITCH < (1 << 31) <= K * (T_PITCH + 16)
    Ad = to_dev_bits(np.ascontiguousarray(A.T), ta, T_PITCH // ESIZE[ta])
    Bd = to_dev_bits(np.ascontiguousarray(B.T), tb, T_PITCH // ESIZE[tb])
    D = out_tensor(M, N, ta == I8)
    Cd = torch.from_numpy(C).to(dev())
    mm.gemm_layout(Ad, Bd, D, True, True, alpha, beta, Cd, a_type=ta, b_type=tb)
    torch.cuda.synchronize()
    Dref, S = oracle.gemm_dense(ta, tb, A, B, alpha, beta, C)
    check(D.cpu().numpy(), Dref, S, ta, K, alpha, beta, C, f"layout max span {ta},{tb}")


@pytest.mark.parametrize("t", [F16, E4M3])
def test_compress_beyond_4gib(t):
    M, K = 600, 1024
    pitch = MAX_PITCH
    A = sparse_a(t, M, K, 21 + t, violate=0.02)
    Ac_ref, idx_ref, bad_ref = oracle.compress24(t, A)
    Ad = to_dev_bits(A, t, pitch // ESIZE[t])
    Ac = to_dev_bits(np.zeros((M, K // 2), oracle.BITS_DTYPE[t]), t, pitch // ESIZE[t])
    assert (M - 1) * pitch >= (1 << 32)
    idxbuf = torch.full((M, pitch // 4), -1, dtype=torch.int32, device=dev())
    idx = idxbuf[:, :(K + 31) // 32]
    bad = torch.zeros(1, dtype=torch.int32, device=dev())
    mm.sparse24_compress(Ad, Ac, idx, bad, a_type=t)
    torch.cuda.synchronize()
    assert np.array_equal(dev_bits_to_host(Ac, t), Ac_ref)
    assert np.array_equal(idx.cpu().numpy().view(np.uint32), idx_ref)
    assert int(bad.item()) == bad_ref
    # nothing written past the index words of a row
    assert bool((idxbuf[:, (K + 31) // 32:(K + 31) // 32 + 64] == -1).all())


@pytest.mark.parametrize("ta,tb", [(F16, F16), (E4M3, E5M2)])
@pytest.mark.parametrize("shape", [None, 256])
def test_sparse_at_max_row_pitch(ta, tb, shape):
    """Compressed A, index, B and D at their largest pitches (the index at 2 Mi words a row)."""
    M, N, K = 300, 260, 1024
    A = sparse_a(ta, M, K, 31 + ta, zero_kept=0.05)
    g = np.random.default_rng(32 + tb)
    B = W.to_bits(g.standard_normal((N, K)) / np.sqrt(K), tb)
    Ac_ref, idx_ref, _ = oracle.compress24(ta, A)
    Acd = to_dev_bits(Ac_ref, ta, max_ld(ta))
    idxbuf = torch.zeros((M, MAX_PITCH // 4), dtype=torch.int32, device=dev())
    idxbuf[:, :idx_ref.shape[1]] = torch.from_numpy(idx_ref.view(np.int32)).to(dev())
    idx = idxbuf[:, :idx_ref.shape[1]]
    Bd = to_dev_bits(B, tb, max_ld(tb))
    D = out_tensor(M, N, False, MAX_PITCH // 4)
    if shape is None:
        mm.gemm_sparse24(Acd, idx, Bd, D, K=K, a_type=ta, b_type=tb)
    else:
        with tile_shape(shape):
            mm.gemm_sparse24(Acd, idx, Bd, D, K=K, a_type=ta, b_type=tb)
    torch.cuda.synchronize()
    Dref, S = oracle.gemm_sparse24(ta, tb, Ac_ref, idx_ref, B)
    assert_close(D.cpu().numpy(), Dref, S, ta, K, 1.0, 0.0, None, f"sparse max pitch {ta},{tb} tile {shape}")
