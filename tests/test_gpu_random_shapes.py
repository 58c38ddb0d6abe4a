"""Randomised shapes against the CPU oracle: dense and 4:2-sparse GEMMs, the skinny (M <= 32)
path, the operand-layout variants and the block-scaled GEMMs, with sizes drawn
from a fixed seed (1..700 rows/columns, K from 1 (dense) or 4 (sparse) to 1200), every
element-type pair, the library's own tile choice, random alpha/beta (beta = 0 included,
int8 with integer alpha/beta) and, for some draws, padded row pitches.  The draws are
fixed, so a failure names a reproducible case."""
import numpy as np
import pytest
import torch

import oracle
import sparse_matrix_multiply_amd as mm
import workloads as W
from gpu_helpers import (assert_close, dev, dev_bits_to_host, out_tensor, padded, to_dev_bits)
from oracle import BF16, E4M3, E5M2, F16, I8

pytestmark = pytest.mark.gpu

PAIRS = [(F16, F16), (BF16, BF16), (I8, I8), (E4M3, E4M3), (E4M3, E5M2), (E5M2, E4M3), (E5M2, E5M2)]


def draw(case, sparse):
    g = np.random.default_rng(9000 + case + (500 if sparse else 0))
    ta, tb = PAIRS[case % len(PAIRS)]
    M, N = (int(x) for x in g.integers(1, 701, size=2))
    K = int(g.integers(1, 301)) * 4 if sparse else int(g.integers(1, 1201))
    if ta == I8:
        alpha, beta = int(g.integers(-3, 4)) or 1, int(g.choice([0, 1, -2]))
    else:
        alpha, beta = float(g.choice([1.0, -0.5, 2.0])), float(g.choice([0.0, 1.0, 0.25]))
    pad = int(g.choice([0, 0, 4, 12]))
    return g, ta, tb, M, N, K, alpha, beta, pad


def host_inputs(g, ta, tb, M, N, K, sparse):
    if ta == I8:
        A = g.integers(-128, 128, size=(M, K)).astype(np.int8)
        B = g.integers(-128, 128, size=(N, K)).astype(np.int8)
        C = g.integers(-1000, 1001, size=(M, N)).astype(np.int32)
    else:
        A = W.to_bits(g.standard_normal((M, K)), ta)
        B = W.to_bits(g.standard_normal((N, K)), tb)
        C = g.standard_normal((M, N)).astype(np.float32)
    if sparse:
        keep = W.prune_mask(M, K, 0, patterns=g.integers(0, 6, size=(M, K // 4)))
        A = np.ascontiguousarray(np.where(keep, A, np.int8(0) if ta == I8 else W.zero_bits(ta)))
    return A, B, C


def check(D, Dref, aux, ta, K, alpha, beta, C, what):
    if ta == I8:
        assert np.array_equal(D, Dref), what
    else:
        assert_close(D, Dref, aux, ta, K, alpha, beta, C if beta != 0 else None, what)


@pytest.mark.parametrize("case", range(28))
def test_random_dense(case):
    g, ta, tb, M, N, K, alpha, beta, pad = draw(case, False)
    A, B, C = host_inputs(g, ta, tb, M, N, K, False)
    es = 2 if ta in (F16, BF16) else 1
    Ad = to_dev_bits(A, ta, padded(K, ta) + pad * (16 // es) // 4 * 4 if pad else None)
    Bd = to_dev_bits(B, tb, padded(K, tb) + pad * (16 // es) // 4 * 4 if pad else None)
    D = out_tensor(M, N, ta == I8, N + pad if pad else None)
    Cd = torch.from_numpy(C).to(dev()) if beta != 0 else None
    mm.gemm_dense(Ad, Bd, D, alpha, beta, Cd, a_type=ta, b_type=tb)
    torch.cuda.synchronize()
    Dref, aux = oracle.gemm_dense(ta, tb, A, B, alpha, beta, C)
    check(D.cpu().numpy(), Dref, aux, ta, K, alpha, beta, C, f"dense case {case}: {ta},{tb} {M}x{N}x{K} "
          f"alpha {alpha} beta {beta} pad {pad}")


@pytest.mark.parametrize("case", range(28))
def test_random_skinny(case):
    """M <= 32 (the skinny kernel: whole-line copies into per-wave LDS rings, a masked last
    chunk): random M 1..32, N 1..700, K 1..5000 (so 0 to 78 whole 128-byte chunks per row),
    padded pitches, every pair."""
    g, ta, tb, _, N, _, alpha, beta, pad = draw(case + 100, False)
    M = int(g.integers(1, 33))
    K = int(g.integers(1, 5001))
    A, B, C = host_inputs(g, ta, tb, M, N, K, False)
    es = 2 if ta in (F16, BF16) else 1
    Ad = to_dev_bits(A, ta, padded(K, ta) + pad * (16 // es) // 4 * 4 if pad else None)
    Bd = to_dev_bits(B, tb, padded(K, tb) + pad * (16 // es) // 4 * 4 if pad else None)
    D = out_tensor(M, N, ta == I8, N + pad if pad else None)
    Cd = torch.from_numpy(C).to(dev()) if beta != 0 else None
    mm.gemm_dense(Ad, Bd, D, alpha, beta, Cd, a_type=ta, b_type=tb)
    torch.cuda.synchronize()
    Dref, aux = oracle.gemm_dense(ta, tb, A, B, alpha, beta, C)
    check(D.cpu().numpy(), Dref, aux, ta, K, alpha, beta, C, f"skinny case {case}: {ta},{tb} {M}x{N}x{K} "
          f"alpha {alpha} beta {beta} pad {pad}")


@pytest.mark.parametrize("case", range(14))
def test_random_sparse(case):
    g, ta, tb, M, N, K, alpha, beta, pad = draw(case, True)
    A, B, C = host_inputs(g, ta, tb, M, N, K, True)
    Ad = to_dev_bits(A, ta)
    Ac = to_dev_bits(np.zeros((M, K // 2), oracle.BITS_DTYPE[ta]), ta)
    idx = torch.zeros((M, (K + 31) // 32), dtype=torch.int32, device=dev())
    mm.sparse24_compress(Ad, Ac, idx, a_type=ta)
    D = out_tensor(M, N, ta == I8, N + pad if pad else None)
    Cd = torch.from_numpy(C).to(dev()) if beta != 0 else None
    mm.gemm_sparse24(Ac, idx, to_dev_bits(B, tb), D, K=K, alpha=alpha, beta=beta, C=Cd, a_type=ta, b_type=tb)
    torch.cuda.synchronize()
    Ac_ref, idx_ref, bad = oracle.compress24(ta, A)
    assert bad == 0
    assert np.array_equal(dev_bits_to_host(Ac, ta), Ac_ref)
    assert np.array_equal(idx.cpu().numpy().view(np.uint32), idx_ref)
    Dref, aux = oracle.gemm_sparse24(ta, tb, Ac_ref, idx_ref, B, alpha, beta, C)
    check(D.cpu().numpy(), Dref, aux, ta, K, alpha, beta, C, f"sparse case {case}: {ta},{tb} {M}x{N}x{K} "
          f"alpha {alpha} beta {beta} pad {pad}")


# ---------------------------------------------------------------- operand layouts --
def to_dev_pitched(bits, pitch_bytes):
    """Host element bits (rows x cols, 1 or 2 bytes each) -> device uint8 rows of pitch_bytes,
    returned as a (rows x cols) view of the right element width."""
    bits = np.ascontiguousarray(bits)
    rows, cols = bits.shape
    es = bits.dtype.itemsize
    buf = torch.zeros((rows, pitch_bytes), dtype=torch.uint8, device=dev())
    buf[:, :cols * es] = torch.from_numpy(bits.view(np.uint8).reshape(rows, cols * es)).to(dev())
    view = buf.view(torch.int16) if es == 2 else buf
    return view[:, :cols]


@pytest.mark.parametrize("case", range(21))
def test_random_layout(case):
    """A stored M-contiguous and / or B stored N-contiguous, every dense pair, random sizes."""
    g, ta, tb, M, N, K, alpha, beta, pad = draw(case, False)
    trans_a, trans_b = [(True, False), (False, True), (True, True)][int(g.integers(0, 3))]
    A, B, C = host_inputs(g, ta, tb, M, N, K, False)
    es = 2 if ta in (F16, BF16) else 1
    pitch = lambda cols: (cols * es + 15) // 16 * 16 + 16 * pad // 4     # noqa: E731
    As = A.T if trans_a else A
    Bs = B.T if trans_b else B
    Ad = to_dev_pitched(As, pitch(As.shape[1]))
    Bd = to_dev_pitched(Bs, pitch(Bs.shape[1]))
    D = out_tensor(M, N, ta == I8, N + pad if pad else None)
    Cd = torch.from_numpy(C).to(dev()) if beta != 0 else None
    mm.gemm_layout(Ad, Bd, D, trans_a, trans_b, alpha, beta, Cd, a_type=ta, b_type=tb)
    torch.cuda.synchronize()
    Dref, aux = oracle.gemm_dense(ta, tb, A, B, alpha, beta, C)
    check(D.cpu().numpy(), Dref, aux, ta, K, alpha, beta, C, f"layout case {case}: {ta},{tb} {M}x{N}x{K} "
          f"trans {trans_a},{trans_b} alpha {alpha} beta {beta} pad {pad}")


# ----------------------------------------------------------------- block-scaled --
MX_PAIRS = [(E4M3, E4M3), (E4M3, E5M2), (E5M2, E4M3), (E5M2, E5M2), (oracle.FP4, oracle.FP4),
            (oracle.FP6, oracle.FP6), (oracle.FP6, oracle.BF6), (oracle.BF6, oracle.FP6), (oracle.BF6, oracle.BF6)]


@pytest.mark.parametrize("case", range(27))
def test_random_mx(case):
    """Block-scaled GEMM: every supported pair, random sizes (K a multiple of 32), random block
    exponents, garbage past K in the scale words, padded pitches."""
    from gpu_helpers import pack_mx_scales
    g = np.random.default_rng(9700 + case)
    ta, tb = MX_PAIRS[case % len(MX_PAIRS)]
    M, N = (int(x) for x in g.integers(1, 701, size=2))
    K = 32 * int(g.integers(1, 41))
    alpha, beta = float(g.choice([1.0, -0.5, 2.0])), float(g.choice([0.0, 1.0, 0.25]))
    pad = int(g.choice([0, 1, 3]))
    packed = ta in (oracle.FP4, oracle.FP6, oracle.BF6)
    if packed:
        bits = 4 if ta == oracle.FP4 else 6
        nbytes = K * bits // 8
        unit = 16 if bits == 4 else 48                  # pitch granule: whole elements, 16-byte rows
        codes = g.integers(0, 1 << bits, size=(M + N, K))
        if bits == 4:
            host = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
        else:
            host = np.packbits(((codes[:, :, None] >> np.arange(6)) & 1).astype(np.uint8).reshape(M + N, -1),
                               axis=1, bitorder="little")
        A, B = host[:M], host[M:]
        pitch = (nbytes + unit - 1) // unit * unit + unit * pad
    else:
        A = W.to_bits(g.standard_normal((M, K)), ta)
        B = W.to_bits(g.standard_normal((N, K)), tb)
        pitch = (K + 15) // 16 * 16 + 16 * pad
    SA = g.integers(110, 145, size=(M, K // 32)).astype(np.uint8)
    SB = g.integers(110, 145, size=(N, K // 32)).astype(np.uint8)
    C = g.standard_normal((M, N)).astype(np.float32)
    D = out_tensor(M, N, False)
    Cd = torch.from_numpy(C).to(dev()) if beta != 0 else None
    mm.gemm_mx(to_dev_pitched(A, pitch), pack_mx_scales(SA, seed=case), to_dev_pitched(B, pitch),
               pack_mx_scales(SB, seed=case + 1), D, alpha, beta, Cd, a_type=ta, b_type=tb)
    torch.cuda.synchronize()
    Dref, S = oracle.gemm_mx(ta, tb, A, SA, B, SB, alpha, beta, C)
    assert_close(D.cpu().numpy(), Dref, S, E4M3, K, alpha, beta, C if beta != 0 else None,
                 f"mx case {case}: {ta},{tb} {M}x{N}x{K} alpha {alpha} beta {beta} pad {pad}")
