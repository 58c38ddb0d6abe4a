"""GPU parity of the split-K calls (mmac_gemm_dense_ws, mmac_gemm_sparse24_ws).

K is cut into ranges that separate workgroups multiply; the last one to finish
a tile sums the partial tiles in range order.  Checked against the oracle for
every element-type pair (int8 bit for bit), with ragged K, beta != 0 (C folded
into range 0's partial), alpha = 0 (C read by the workgroup that finishes),
the epilogue variants, forced range counts 2-4 on every tile shape, and the
automatic plan on small outputs with a long K.  Also: repeated calls
give identical bits, small-integer products equal the oracle exactly, the
tile counters are zero again after every call, and a workspace that is too
small falls back to the unsplit kernel.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_matrix_multiply_amd as mm
import workloads as W
from gpu_helpers import assert_close, compress_dev, dev, env, out_tensor, sample_entries, to_dev_bits
from oracle import BF16, E4M3, E5M2, F16, I8

pytestmark = pytest.mark.gpu

PAIRS = [(BF16, BF16), (F16, F16), (I8, I8), (E4M3, E4M3), (E4M3, E5M2), (E5M2, E4M3), (E5M2, E5M2)]


def inputs(ta, tb, M, N, K, seed):
    g = np.random.default_rng(seed)
    if ta == I8:
        A = g.integers(-128, 128, size=(M, K)).astype(np.int8)
        B = g.integers(-128, 128, size=(N, K)).astype(np.int8)
        C = g.integers(-1000, 1001, size=(M, N)).astype(np.int32)
        return A, B, C, 1, 3
    A = W.to_bits(g.standard_normal((M, K)), ta)
    B = W.to_bits(g.standard_normal((N, K)), tb)
    C = g.standard_normal((M, N)).astype(np.float32)
    return A, B, C, 1.25, -0.5


def counters_zero(ws, M, N, tile=256):
    tiles = ((M + tile - 1) // tile) * ((N + tile - 1) // tile)
    return int(torch.count_nonzero(ws[:tiles * 4]).item()) == 0


def run(ta, tb, A, B, alpha, beta, C, ws, sparse=False, D=None):
    M, K = A.shape
    N = B.shape[0]
    integer = ta == I8
    if D is None:
        D = out_tensor(M, N, integer)
    Cd = torch.from_numpy(np.ascontiguousarray(C)).to(dev()) if beta != 0 else None
    Bd = to_dev_bits(B, tb)
    if sparse:
        Acd, idxd, _ = compress_dev(ta, to_dev_bits(A, ta), M, K, prune=True)
        mm.gemm_sparse24(Acd, idxd, Bd, D, K=K, alpha=alpha, beta=beta, C=Cd, a_type=ta, b_type=tb, workspace=ws)
    else:
        mm.gemm_dense(to_dev_bits(A, ta), Bd, D, alpha, beta, Cd, a_type=ta, b_type=tb, workspace=ws)
    torch.cuda.synchronize()
    return D


def oracle_ref(sparse, ta, tb, A, B, alpha, beta, C):
    if sparse:
        Ac, idx, _ = oracle.prune_compress24(ta, A)
        return oracle.gemm_sparse24(ta, tb, Ac, idx, B, alpha, beta, C if beta else None)
    return oracle.gemm_dense(ta, tb, A, B, alpha, beta, C if beta else None)


@pytest.mark.parametrize("sparse", [False, True])
@pytest.mark.parametrize("ta,tb", PAIRS)
@pytest.mark.parametrize("splits", [2, 3, 4])
@pytest.mark.parametrize("tile", [256, 128, 64])
def test_forced_splits_match_oracle(sparse, ta, tb, splits, tile):
    M, N, K = 300, 260, 1000
    A, B, C, alpha, beta = inputs(ta, tb, M, N, K, splits * 13 + tile + ta * 7 + tb + sparse)
    with env(MMAC_SPLITK=splits, MMAC_TILE=tile):
        ws = mm.workspace(ta, M, N, K, sparse=sparse)
        assert ws is not None
        D1 = run(ta, tb, A, B, alpha, beta, C, ws, sparse).cpu().numpy()
        assert counters_zero(ws, M, N, tile)
        D2 = run(ta, tb, A, B, alpha, beta, C, ws, sparse).cpu().numpy()
    assert np.array_equal(D1.view(np.uint32), D2.view(np.uint32)), "repeated split calls differ"
    Dref, aux = oracle_ref(sparse, ta, tb, A, B, alpha, beta, C)
    if ta == I8:
        assert np.array_equal(D1, Dref)
    else:
        assert_close(D1, Dref, aux, ta, K, alpha, beta, C, f"splits {splits} tile {tile}")


@pytest.mark.parametrize("sparse", [False, True])
@pytest.mark.parametrize("ta,tb", [(BF16, BF16), (F16, F16), (E4M3, E5M2)])
def test_small_integers_exact_across_splits(sparse, ta, tb):
    """Every partial sum is an integer below 2^24: all range counts give the oracle's bits."""
    M, N, K = 200, 300, 2048
    g = np.random.default_rng(ta + 3 * tb)
    A = W.to_bits(g.integers(-4, 5, size=(M, K)).astype(np.float64), ta)
    B = W.to_bits(g.integers(-4, 5, size=(N, K)).astype(np.float64), tb)
    C = g.integers(-50, 51, size=(M, N)).astype(np.float32)
    Dref, _ = oracle_ref(sparse, ta, tb, A, B, 1.0, 1.0, C)
    for splits in (1, 2, 3, 4):
        with env(MMAC_SPLITK=splits, MMAC_TILE=256):
            ws = mm.workspace(ta, M, N, K, sparse=sparse)
            if splits > 1:
                assert ws is not None
            D = run(ta, tb, A, B, 1.0, 1.0, C, ws, sparse).cpu().numpy()
        assert np.array_equal(D.astype(np.float64), Dref), f"splits {splits}"


@pytest.mark.parametrize("ta", [BF16, I8])
def test_alpha_zero_reads_c_once(ta):
    """alpha = 0 with a split: D = beta * C exactly (C read by the finishing workgroup only)."""
    M, N, K = 260, 270, 1024
    A, B, C, _, _ = inputs(ta, ta, M, N, K, 4)
    with env(MMAC_SPLITK=2, MMAC_TILE=256):
        ws = mm.workspace(ta, M, N, K)
        D = run(ta, ta, A, B, 0, 2, C, ws).cpu().numpy()
    assert np.array_equal(D, (2 * C).astype(D.dtype))


@pytest.mark.parametrize("sparse", [False, True])
@pytest.mark.parametrize("d_type,tdt,oout", [(mm.OUT_BF16, torch.bfloat16, oracle.OUT_BF16),
                                             (mm.OUT_F16, torch.float16, oracle.OUT_F16)])
def test_epilogue_variants_with_splits(sparse, d_type, tdt, oout):
    """bfloat16 / binary16 C and D, bias and ReLU after the split sum: exact on integer products."""
    ta = tb = E4M3
    M, N, K = 300, 200, 1536
    g = np.random.default_rng(d_type + 5 * sparse)
    A = W.to_bits(g.integers(-4, 5, size=(M, K)).astype(np.float64), ta)
    B = W.to_bits(g.integers(-4, 5, size=(N, K)).astype(np.float64), tb)
    C = g.integers(-64, 65, size=(M, N)).astype(np.float32)
    bias = g.integers(-300, 301, size=N).astype(np.float32)
    Y, _ = oracle_ref(sparse, ta, tb, A, B, 1.0, 1.0, C)
    ref, _ = oracle.epilogue(Y, bias, mm.ACT_RELU, oout)
    Cd = torch.from_numpy(C).to(dev()).to(tdt)
    D = torch.full((M, N), float("nan"), dtype=tdt, device=dev())
    with env(MMAC_SPLITK=3, MMAC_TILE=256):
        ws = mm.workspace(ta, M, N, K, sparse=sparse)
        Bd = to_dev_bits(B, tb)
        bd = torch.from_numpy(bias).to(dev())
        if sparse:
            Acd, idxd, _ = compress_dev(ta, to_dev_bits(A, ta), M, K, prune=True)
            mm.gemm_sparse24(Acd, idxd, Bd, D, K=K, alpha=1.0, beta=1.0, C=Cd, a_type=ta, b_type=tb, bias=bd,
                             act=mm.ACT_RELU, workspace=ws)
        else:
            mm.gemm_dense(to_dev_bits(A, ta), Bd, D, 1.0, 1.0, Cd, a_type=ta, b_type=tb, bias=bd, act=mm.ACT_RELU,
                          workspace=ws)
        torch.cuda.synchronize()
    got = D.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_too_small_workspace_runs_unsplit():
    ta = tb = BF16
    M, N, K = 300, 260, 1000
    A, B, C, alpha, beta = inputs(ta, tb, M, N, K, 8)
    with env(MMAC_SPLITK=2, MMAC_TILE=256):
        need = mm.workspace_bytes(ta, M, N, K)
        ws = torch.zeros(need - 16, dtype=torch.uint8, device=dev())
        D = run(ta, tb, A, B, alpha, beta, C, ws).cpu().numpy()
        assert int(torch.count_nonzero(ws).item()) == 0          # not touched
    with env(MMAC_TILE=256):
        D0 = run(ta, tb, A, B, alpha, beta, C, None).cpu().numpy()
    assert np.array_equal(D.view(np.uint32), D0.view(np.uint32))


@pytest.mark.parametrize("ta,tb,M,N,K,sparse,splits", [(BF16, BF16, 512, 512, 16384, False, 4),
                                                        (E4M3, E5M2, 512, 512, 16384, False, 4),
                                                        (E4M3, E4M3, 1024, 512, 8192, True, 2)])
def test_automatic_split(ta, tb, M, N, K, sparse, splits):
    """Small outputs with a long K: the library splits K on its own (64 x 64 tiles, 64 or 128 of
    them, into 4 or 2 ranges); sampled against the oracle, including two whole 256 x 256 blocks."""
    tiles = (M // 64) * (N // 64)
    assert mm.workspace_bytes(ta, M, N, K, sparse) == (tiles * 4 + 255) // 256 * 256 + splits * tiles * 64 * 64 * 4
    g = np.random.default_rng(M + K + sparse)
    A = W.to_bits(g.standard_normal((M, K)), ta)
    B = W.to_bits(g.standard_normal((N, K)), tb)
    C = g.standard_normal((M, N)).astype(np.float32)
    alpha, beta = 0.5, 1.0
    ws = mm.workspace(ta, M, N, K, sparse=sparse)
    D = run(ta, tb, A, B, alpha, beta, C, ws, sparse)
    assert counters_zero(ws, M, N, 64)
    if sparse:
        Ac, idx, _ = oracle.prune_compress24(ta, A)
        fn = lambda ii, jj: oracle.gemm_sparse24_entries(ta, tb, Ac, idx, B, ii, jj, alpha, beta, C)
    else:
        fn = lambda ii, jj: oracle.gemm_dense_entries(ta, tb, A, B, ii, jj, alpha, beta, C)
    ii, jj = sample_entries(M, N, 4000, 12, tiles=((0, 0), ((M - 1) // 256, (N - 1) // 256)))
    ref, S = fn(ii, jj)
    got = D[torch.from_numpy(ii).to(dev()), torch.from_numpy(jj).to(dev())].cpu().numpy()
    assert_close(got, ref, S, ta, K, alpha, beta, C[ii, jj], f"{M}x{N}x{K}")
    # the same product unsplit: equal up to summation order
    D0 = run(ta, tb, A, B, alpha, beta, C, None, sparse)
    got0 = D0[torch.from_numpy(ii).to(dev()), torch.from_numpy(jj).to(dev())].cpu().numpy()
    assert_close(got0, ref, S, ta, K, alpha, beta, C[ii, jj], "unsplit")


def test_share_shape_is_not_split():
    """One GPU's 8192 x 1024 x 8192 share already has a tile per compute unit (128 x 256 tiles)."""
    assert mm.workspace_bytes(BF16, 8192, 1024, 8192) == 0
    assert mm.workspace_bytes(E4M3, 8192, 1024, 8192, True) == 0


@pytest.mark.parametrize("alpha,beta,a_zero", [(2.0 ** -100, 2.0 ** 100, False), (2.0 ** 100, 2.0 ** -100, True),
                                               (1e-39, 1.0, False)])
@pytest.mark.parametrize("ta,tb", [(BF16, BF16), (E4M3, E5M2)])
def test_extreme_alpha_beta_ratios_split(ta, tb, alpha, beta, a_zero):
    """The same scale pairs under a forced split into three ranges (C then reaches the result in
    the workgroup that finishes the tile, or in range 0's partial)."""
    M, N, K = 300, 260, 1000
    A, B, C, _, _ = inputs(ta, tb, M, N, K, 41)
    if a_zero:
        A = np.zeros_like(A)
    with env(MMAC_SPLITK=3, MMAC_TILE=64):
        ws = mm.workspace(ta, M, N, K)
        assert ws is not None
        D = run(ta, tb, A, B, alpha, beta, C, ws).cpu().numpy()
        assert counters_zero(ws, M, N, 64)
    a32, b32 = float(np.float32(alpha)), float(np.float32(beta))
    Dref, S = oracle.gemm_dense(ta, tb, A, B, a32, b32, C)
    assert_close(D, Dref, S, ta, K, a32, b32, C, f"split alpha {alpha} beta {beta}")
    if a_zero:
        assert np.array_equal(D.astype(np.float64), Dref)
