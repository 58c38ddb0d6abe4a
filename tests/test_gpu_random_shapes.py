"""Randomised shapes against the CPU oracle: dense and 4:2-sparse GEMMs with sizes drawn
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
