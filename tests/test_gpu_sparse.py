"""GPU parity of mmac_sparse24_compress and mmac_gemm_sparse24 against the CPU oracle.

- compressor: bit-exact Ac and index words (and the violation count) for every
  element type, ragged K (partial 16-byte units and partial index words),
  zero-heavy and violating groups;
- sparse GEMM: every supported pair and tile shape, all six 2-of-4 patterns,
  ragged tails, exact small-integer inputs, and the GPU compressor feeding
  the GPU sparse GEMM.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_matrix_multiply_amd as mm
import workloads as W
from gpu_helpers import (assert_close, compress_dev, dev, dev_bits_to_host, out_tensor, tile_shape,
                         to_dev_bits)
from oracle import BF16, E4M3, E5M2, F16, I8

pytestmark = pytest.mark.gpu

TYPES = [F16, BF16, I8, E4M3, E5M2]
PAIRS = [(F16, F16), (BF16, BF16), (I8, I8), (E4M3, E4M3), (E4M3, E5M2), (E5M2, E4M3), (E5M2, E5M2)]


def sparse_a(t, M, K, seed, violate=0.0, zero_kept=0.0):
    """A 4:2 matrix with uniform patterns; optionally some groups get a third non-zero
    and some kept values are zeroed (groups with fewer than two non-zeros)."""
    g = np.random.default_rng(seed)
    pats = g.integers(0, 6, size=(M, K // 4))
    keep = W.prune_mask(M, K, 0, patterns=pats)
    if t == I8:
        vals = g.integers(1, 128, size=(M, K)) * np.where(g.random((M, K)) < 0.5, -1, 1)
        dense = vals.astype(np.int8)
        zero = np.int8(0)
    else:
        dense = W.to_bits(g.standard_normal((M, K)) + np.sign(g.standard_normal((M, K))) * 0.25, t)
        zero = W.zero_bits(t)
    if violate:
        keep |= (g.random((M, K)) < violate)
    if zero_kept:
        keep &= ~(g.random((M, K)) < zero_kept)
    return np.ascontiguousarray(np.where(keep, dense, zero))


@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("M,K", [(1, 4), (3, 12), (64, 64), (77, 200), (130, 1028), (9, 4100)])
def test_compress_bit_exact(t, M, K):
    A = sparse_a(t, M, K, M + K + t, violate=0.05, zero_kept=0.1)
    Ac_ref, idx_ref, bad_ref = oracle.compress24(t, A)
    Ac, idx, bad = compress_dev(t, to_dev_bits(A, t), M, K)
    torch.cuda.synchronize()
    assert np.array_equal(dev_bits_to_host(Ac, t), Ac_ref)
    assert np.array_equal(idx.cpu().numpy().view(np.uint32), idx_ref)
    assert int(bad.item()) == bad_ref


@pytest.mark.parametrize("t", [F16, E4M3])
def test_compress_special_values(t):
    """Signed zeros, NaN (counts as non-zero) and all-zero groups."""
    M, K = 8, 64
    if t == F16:
        alphabet = np.array([0x0000, 0x8000, 0x3C00, 0xBC00, 0x7E00], np.uint16)
    else:
        alphabet = np.array([0x00, 0x80, 0x38, 0xB8, 0x7F], np.uint8)
    A = alphabet[np.random.default_rng(1).integers(0, 5, size=(M, K))]
    Ac_ref, idx_ref, bad_ref = oracle.compress24(t, A)
    Ac, idx, bad = compress_dev(t, to_dev_bits(A, t), M, K)
    torch.cuda.synchronize()
    assert np.array_equal(dev_bits_to_host(Ac, t), Ac_ref)
    assert np.array_equal(idx.cpu().numpy().view(np.uint32), idx_ref)
    assert int(bad.item()) == bad_ref


def run_sparse(ta, tb, Ac, idx, B, K, alpha, beta, C):
    M, N = Ac.shape[0], B.shape[0]
    Acd, Bd = to_dev_bits(Ac, ta), to_dev_bits(B, tb)
    idxd = torch.from_numpy(np.ascontiguousarray(idx).view(np.int32)).to(dev())
    D = out_tensor(M, N, ta == I8)
    Cd = torch.from_numpy(np.ascontiguousarray(C)).to(dev()) if beta != 0 else None
    mm.gemm_sparse24(Acd, idxd, Bd, D, K=K, alpha=alpha, beta=beta, C=Cd, a_type=ta, b_type=tb)
    torch.cuda.synchronize()
    return D.cpu().numpy()


def b_and_c(tb, N, M, K, seed):
    g = np.random.default_rng(seed)
    if tb == I8:
        return (g.integers(-128, 128, size=(N, K)).astype(np.int8),
                g.integers(-1000, 1001, size=(M, N)).astype(np.int32), 2, -3)
    return W.to_bits(g.standard_normal((N, K)), tb), g.standard_normal((M, N)).astype(np.float32), 1.25, 0.5


@pytest.mark.parametrize("tile", [256, 2561, 1282, 128, 64])
@pytest.mark.parametrize("ta,tb", PAIRS)
@pytest.mark.parametrize("M,N,K", [(64, 64, 64), (100, 77, 200), (257, 130, 332), (40, 300, 1028)])
def test_sparse_matches_oracle(ta, tb, M, N, K, tile):
    A = sparse_a(ta, M, K, M + N + K + ta)
    Ac, idx, bad = oracle.compress24(ta, A)
    assert bad == 0
    B, C, alpha, beta = b_and_c(tb, N, M, K, K + tb)
    with tile_shape(tile):
        D = run_sparse(ta, tb, Ac, idx, B, K, alpha, beta, C)
    Dref, aux = oracle.gemm_sparse24(ta, tb, Ac, idx, B, alpha, beta, C)
    if ta == I8:
        assert np.array_equal(D, Dref)
    else:
        assert_close(D, Dref, aux, ta, K, alpha, beta, C, f"sparse {ta},{tb} {M}x{N}x{K} tile {tile}")


@pytest.mark.parametrize("ta,tb", [(F16, F16), (BF16, BF16), (E4M3, E5M2), (I8, I8)])
@pytest.mark.parametrize("pattern", range(6))
def test_each_pattern_exact(ta, tb, pattern):
    """One pattern everywhere, small integers: exact results, so every nibble value the
    compressor can write must select exactly the right B rows."""
    M, N, K = 64, 64, 256
    g = np.random.default_rng(pattern)
    keep = W.prune_mask(M, K, 0, patterns=np.full((M, K // 4), pattern))
    if ta == I8:
        A = np.where(keep, g.integers(1, 5, size=(M, K)), 0).astype(np.int8)
        B = g.integers(-4, 5, size=(N, K)).astype(np.int8)
    else:
        A = np.where(keep, W.to_bits(g.integers(1, 5, size=(M, K)).astype(np.float64), ta), W.zero_bits(ta))
        B = W.to_bits(g.integers(-4, 5, size=(N, K)).astype(np.float64), tb)
    Ac, idx, _ = oracle.compress24(ta, A)
    C = np.zeros((M, N), np.int32 if ta == I8 else np.float32)
    D = run_sparse(ta, tb, Ac, idx, B, K, 1, 0, C)
    Dref, _ = oracle.gemm_sparse24(ta, tb, Ac, idx, B, 1, 0, C)
    assert np.array_equal(D.astype(np.float64), np.asarray(Dref, np.float64))


@pytest.mark.parametrize("ta,tb", [(F16, F16), (E4M3, E5M2)])
def test_gpu_compress_feeds_gpu_sparse_gemm(ta, tb):
    M, N, K = 300, 200, 512
    A = sparse_a(ta, M, K, 11, zero_kept=0.02)
    B, C, alpha, beta = b_and_c(tb, N, M, K, 12)
    Acd, idxd, bad = compress_dev(ta, to_dev_bits(A, ta), M, K)
    D = out_tensor(M, N, False)
    mm.gemm_sparse24(Acd, idxd, to_dev_bits(B, tb), D, K=K, alpha=alpha, beta=beta,
                     C=torch.from_numpy(C).to(dev()), a_type=ta, b_type=tb)
    torch.cuda.synchronize()
    Ddense, S = oracle.gemm_dense(ta, tb, A, B, alpha, beta, C)
    assert_close(D.cpu().numpy(), Ddense, S, ta, K, alpha, beta, C)


# ---------------------------------------------------- magnitude prune + compress --

PRUNE_ALPHABET = {
    F16: [0x0000, 0x8000, 0x3C00, 0xBC00, 0x4000, 0xC000, 0x7C00, 0xFC00, 0x7E00, 0x7C01, 0x0001],
    BF16: [0x0000, 0x8000, 0x3F80, 0xBF80, 0x4000, 0xC000, 0x7F80, 0xFF80, 0x7FC0, 0xFF81, 0x0001],
    E4M3: [0x00, 0x80, 0x38, 0xB8, 0x40, 0xC0, 0x7E, 0xFE, 0x7F, 0xFF, 0x01],
    E5M2: [0x00, 0x80, 0x3C, 0xBC, 0x40, 0xC0, 0x7C, 0xFC, 0x7E, 0x7D, 0x01],
    I8: [0, 1, -1, 2, -2, 127, -127, -128, 64, -64, 3],
}


def dense_a(t, M, K, seed):
    """Dense A (no pattern): normal values with some exact zeros and repeated magnitudes."""
    g = np.random.default_rng(seed)
    if t == I8:
        A = g.integers(-128, 128, size=(M, K)).astype(np.int8)
    else:
        A = W.to_bits(np.round(g.standard_normal((M, K)) * 8) / 8, t)   # many equal magnitudes
    zero = np.int8(0) if t == I8 else W.zero_bits(t)
    return np.ascontiguousarray(np.where(g.random((M, K)) < 0.1, zero, A))


@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("M,K", [(1, 4), (3, 12), (64, 64), (77, 200), (130, 1028), (9, 4100)])
def test_prune_compress_bit_exact(t, M, K):
    A = dense_a(t, M, K, 3 * M + K + t)
    Ac_ref, idx_ref, bad_ref = oracle.prune_compress24(t, A)
    Ac, idx, bad = compress_dev(t, to_dev_bits(A, t), M, K, prune=True)
    torch.cuda.synchronize()
    assert np.array_equal(dev_bits_to_host(Ac, t), Ac_ref)
    assert np.array_equal(idx.cpu().numpy().view(np.uint32), idx_ref)
    assert int(bad.item()) == bad_ref


@pytest.mark.parametrize("t", TYPES)
def test_prune_compress_special_values(t):
    """Ties, signed zeros, infinities, every NaN payload, int8 -128."""
    M, K = 16, 4 * 96
    alpha = np.array(PRUNE_ALPHABET[t], oracle.BITS_DTYPE[t])
    A = alpha[np.random.default_rng(t).integers(0, len(alpha), size=(M, K))]
    Ac_ref, idx_ref, bad_ref = oracle.prune_compress24(t, A)
    Ac, idx, bad = compress_dev(t, to_dev_bits(A, t), M, K, prune=True)
    torch.cuda.synchronize()
    assert np.array_equal(dev_bits_to_host(Ac, t), Ac_ref)
    assert np.array_equal(idx.cpu().numpy().view(np.uint32), idx_ref)
    assert int(bad.item()) == bad_ref


@pytest.mark.parametrize("t", [F16, E4M3])
def test_prune_compress_equals_compress_on_4_2_input(t):
    M, K = 100, 520
    A = sparse_a(t, M, K, 21, zero_kept=0.1)
    got = compress_dev(t, to_dev_bits(A, t), M, K, prune=True)
    want = compress_dev(t, to_dev_bits(A, t), M, K, prune=False)
    torch.cuda.synchronize()
    assert np.array_equal(dev_bits_to_host(got[0], t), dev_bits_to_host(want[0], t))
    assert torch.equal(got[1].cpu(), want[1].cpu()) and int(got[2].item()) == int(want[2].item()) == 0


@pytest.mark.parametrize("ta,tb", [(F16, F16), (BF16, BF16), (E4M3, E5M2), (I8, I8)])
def test_gpu_prune_compress_feeds_gpu_sparse_gemm(ta, tb):
    """Dense A -> GPU prune+compress -> GPU sparse GEMM, against the oracle's dense GEMM of the
    pruned matrix (the oracle's pruning, decompressed)."""
    M, N, K = 200, 136, 640
    A = dense_a(ta, M, K, 5)
    B, C, alpha, beta = b_and_c(tb, N, M, K, 6)
    Acd, idxd, _ = compress_dev(ta, to_dev_bits(A, ta), M, K, prune=True)
    D = out_tensor(M, N, ta == I8)
    Cd = torch.from_numpy(C).to(dev())
    mm.gemm_sparse24(Acd, idxd, to_dev_bits(B, tb), D, K=K, alpha=alpha, beta=beta, C=Cd, a_type=ta, b_type=tb)
    torch.cuda.synchronize()
    Ac_ref, idx_ref, _ = oracle.prune_compress24(ta, A)
    Apruned = oracle.decompress24(ta, Ac_ref, idx_ref, K)
    Dref, aux = oracle.gemm_dense(ta, tb, Apruned, B, alpha, beta, C)
    if ta == I8:
        assert np.array_equal(D.cpu().numpy(), Dref)
    else:
        assert_close(D.cpu().numpy(), Dref, aux, ta, K, alpha, beta, C, f"pruned {ta},{tb}")
