"""GPU parity for infinities and NaNs in the operands (dense and 4:2 sparse).

IEEE arithmetic fixes the outcome of every sum that meets a special value, whatever
the order of summation: a NaN operand, inf * 0, or +inf and -inf in one sum give NaN;
otherwise an infinite product gives an infinity of its sign.  The oracle sums in fp64,
the GPU in fp32 inside the matrix instructions; each output must have the oracle's
class (NaN, +inf, -inf, finite), and the finite outputs must pass the usual gate.
The specials are planted in a few rows of A and columns of B; zeros are planted where
they meet an infinity.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import sparse_matrix_multiply_amd as mm
from gpu_helpers import assert_close, compress_dev, dev, out_tensor, run_dense, to_dev_bits
from oracle import BF16, E4M3, E5M2, F16

pytestmark = pytest.mark.gpu


# (+inf, -inf, NaN) bit codes; E4M3 has no infinity, NaN stands in for it there
SPECIAL = {BF16: (0x7F80, 0xFF80, 0x7FC0), F16: (0x7C00, 0xFC00, 0x7E00), E5M2: (0x7C, 0xFC, 0x7E),
           E4M3: (0x7F, 0xFF, 0x7F)}


def planted(ta, tb, M, N, K, seed, sparse=False):
    g = np.random.default_rng(seed)
    A = g.standard_normal((M, K))
    B = g.standard_normal((N, K))
    if sparse:                                    # 4:2 pattern: keep positions {0, 2} of each group
        A[:, 1::4] = 0.0
        A[:, 3::4] = 0.0
    A[9, 40] = 0.0                                # row 9 meets column 2's -inf with a zero: NaN in (9, 2)
    B[4, 8] = 0.0                                 # column 4 meets row 3's +inf with a zero: NaN in (3, 4)
    A, B = W.to_bits(A, ta), W.to_bits(B, tb)
    pa, na, nan_a = SPECIAL[ta]
    pb, nb, _ = SPECIAL[tb]
    A[3, 8] = pa                                  # row 3: +inf at k = 8
    A[5, 16] = nan_a                              # row 5: NaN
    A[7, 24] = na                                 # row 7: -inf and +inf: NaN wherever both meet non-zeros
    A[7, 32] = pa
    B[2, 40] = nb                                 # column 2: -inf at k = 40
    return A, B


def classes(x):
    x = np.asarray(x, np.float64)
    return np.where(np.isnan(x), 3, np.where(np.isposinf(x), 1, np.where(np.isneginf(x), 2, 0)))


def check(D, Dref, S, t, K, what):
    cg, cr = classes(D), classes(Dref)
    bad = np.argwhere(cg != cr)
    assert bad.size == 0, f"{what}: class mismatch at {bad[:5].tolist()}: gpu {cg[tuple(bad[0])]} ref {cr[tuple(bad[0])]}"
    assert (cr != 0).sum() >= 4, "the planted specials must reach the output"
    fin = cr == 0
    D2, R2, S2 = np.where(fin, D, 0.0), np.where(fin, Dref, 0.0), np.where(fin, S, 0.0)
    assert_close(D2, R2, S2, t, K, 1.0, 0.0, None, what)


@pytest.mark.parametrize("ta,tb", [(BF16, BF16), (F16, F16), (E4M3, E5M2), (E5M2, E5M2), (E4M3, E4M3)])
@pytest.mark.parametrize("M", [12, 100])                  # skinny and tiled kernels
def test_dense_specials(ta, tb, M):
    N, K = 40, 96
    A, B = planted(ta, tb, M, N, K, M + ta)
    D = run_dense(ta, tb, A, B, 1.0, 0.0, None)
    with np.errstate(invalid="ignore"):
        Dref, S = oracle.gemm_dense(ta, tb, A, B)
    check(D, Dref, S, ta, K, f"dense {ta},{tb} M={M}")


@pytest.mark.parametrize("ta,tb", [(BF16, BF16), (E5M2, E5M2), (E4M3, E5M2)])
def test_sparse_specials(ta, tb):
    M, N, K = 100, 40, 96
    A, B = planted(ta, tb, M, N, K, 7 + ta, sparse=True)
    Ac, idx, bad = oracle.compress24(ta, A)
    assert bad == 0
    Acd, idxd, badd = compress_dev(ta, to_dev_bits(A, ta), M, K)
    torch.cuda.synchronize()
    assert int(badd.item()) == 0
    D = out_tensor(M, N, False)
    mm.gemm_sparse24(Acd, idxd, to_dev_bits(B, tb), D, K=K, a_type=ta, b_type=tb)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore"):
        Dref, S = oracle.gemm_sparse24(ta, tb, Ac, idx, B)
    check(D.cpu().numpy(), Dref, S, ta, K, f"sparse {ta},{tb}")
