"""GPU parity of mmac_gemm_dense against the CPU oracle (small and ragged shapes).

Every supported element-type pair, every tile shape the library can pick,
shapes that span several tiles with ragged M, N and K tails (including K tails
that cut a 16-byte unit), exact small-integer inputs (bit-exact whatever the
summation order), the beta = 0 / NaN-C rule, in-place C == D, K == 0, and
run-to-run determinism.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_matrix_multiply_amd as mm
import workloads as W
from gpu_helpers import (FP8, assert_close, dev, out_tensor, run_dense, tile_shape, to_dev_bits)
from oracle import BF16, E4M3, E5M2, F16, I8

pytestmark = pytest.mark.gpu

PAIRS = [(BF16, BF16), (F16, F16), (I8, I8), (E4M3, E4M3), (E4M3, E5M2), (E5M2, E4M3), (E5M2, E5M2)]
SHAPES = [(64, 64, 64), (100, 77, 200), (257, 130, 333), (33, 300, 1000), (300, 260, 128), (1, 1, 1)]


def inputs(ta, tb, M, N, K, seed):
    g = np.random.default_rng(seed)
    if ta == I8:
        A = g.integers(-128, 128, size=(M, K)).astype(np.int8)
        B = g.integers(-128, 128, size=(N, K)).astype(np.int8)
        C = g.integers(-1000, 1001, size=(M, N)).astype(np.int32)
        return A, B, C, 3, -2
    A = W.to_bits(g.standard_normal((M, K)), ta)
    B = W.to_bits(g.standard_normal((N, K)), tb)
    C = g.standard_normal((M, N)).astype(np.float32)
    return A, B, C, 1.5, -0.75


@pytest.mark.parametrize("tile", [256, 2561, 1282, 128, 64])
@pytest.mark.parametrize("ta,tb", PAIRS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_dense_matches_oracle(ta, tb, M, N, K, tile):
    A, B, C, alpha, beta = inputs(ta, tb, M, N, K, M * 7 + N * 3 + K + ta * 11 + tb)
    with tile_shape(tile):
        D = run_dense(ta, tb, A, B, alpha, beta, C)
    Dref, aux = oracle.gemm_dense(ta, tb, A, B, alpha, beta, C)
    if ta == I8:
        assert np.array_equal(D, Dref), f"int8 mismatch at {np.argwhere(D != Dref)[:5]}"
    else:
        assert_close(D, Dref, aux, ta, K, alpha, beta, C, f"{ta},{tb} {M}x{N}x{K} tile {tile}")


@pytest.mark.parametrize("ta,tb", [(BF16, BF16), (F16, F16), (E4M3, E5M2), (E5M2, E5M2)])
def test_small_integers_are_exact(ta, tb):
    """|a|, |b| <= 4 integers with K = 520: every partial sum is an integer below 2^24,
    so the fp32 result is exact whatever the order of summation."""
    M, N, K = 130, 70, 520
    g = np.random.default_rng(5)
    A = W.to_bits(g.integers(-4, 5, size=(M, K)).astype(np.float64), ta)
    B = W.to_bits(g.integers(-4, 5, size=(N, K)).astype(np.float64), tb)
    C = g.integers(-50, 51, size=(M, N)).astype(np.float32)
    for tile in (256, 64):
        with tile_shape(tile):
            D = run_dense(ta, tb, A, B, 1.0, 1.0, C)
        Dref, _ = oracle.gemm_dense(ta, tb, A, B, 1.0, 1.0, C)
        assert np.array_equal(D.astype(np.float64), Dref)


@pytest.mark.parametrize("t", [BF16, E4M3])
def test_identity_and_permutation(t):
    n = 160
    one, zero = W.to_bits(np.ones(1), t)[0], W.zero_bits(t)
    g = np.random.default_rng(3)
    B = W.to_bits(g.standard_normal((n, n)), t)
    perm = g.permutation(n)
    P = np.full((n, n), zero, oracle.BITS_DTYPE[t])
    P[np.arange(n), perm] = one
    D = run_dense(t, t, P, B, 1.0, 0.0, None)
    Bf = W.from_bits(B, t).astype(np.float64)          # Bf[j, k] = B[k, j]
    assert np.array_equal(D.astype(np.float64), Bf.T[perm, :])


def test_beta_zero_never_reads_c():
    M, N, K = 96, 96, 64
    A, B, _, _, _ = inputs(BF16, BF16, M, N, K, 1)
    Cnan = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev())
    D = run_dense(BF16, BF16, A, B, 1.0, 0.0, None, C_dev=Cnan)
    assert np.isfinite(D).all()
    Dref, S = oracle.gemm_dense(BF16, BF16, A, B)
    assert_close(D, Dref, S, BF16, K, 1.0, 0.0)


@pytest.mark.parametrize("ta", [BF16, I8])
def test_in_place_c_equals_d(ta):
    M, N, K = 200, 144, 96
    A, B, C, alpha, beta = inputs(ta, ta, M, N, K, 2)
    Cd = torch.from_numpy(C).to(dev())
    mm.gemm_dense(to_dev_bits(A, ta), to_dev_bits(B, ta), Cd, alpha, beta, Cd, a_type=ta, b_type=ta)
    torch.cuda.synchronize()
    Dref, aux = oracle.gemm_dense(ta, ta, A, B, alpha, beta, C)
    if ta == I8:
        assert np.array_equal(Cd.cpu().numpy(), Dref)
    else:
        assert_close(Cd.cpu().numpy(), Dref, aux, ta, K, alpha, beta, C)


def test_k_zero_gives_beta_c():
    M, N = 70, 90
    C = np.random.default_rng(1).standard_normal((M, N)).astype(np.float32)
    Ad = to_dev_bits(np.zeros((M, 8), np.uint16), BF16)[:, :0]
    Bd = to_dev_bits(np.zeros((N, 8), np.uint16), BF16)[:, :0]
    D = out_tensor(M, N, False)
    mm.gemm_dense(Ad, Bd, D, 2.0, 0.5, torch.from_numpy(C).to(dev()), a_type=BF16, b_type=BF16)
    torch.cuda.synchronize()
    assert np.array_equal(D.cpu().numpy(), (np.float32(0.5) * C))


@pytest.mark.parametrize("tile", [256, 64])
@pytest.mark.parametrize("ldd,first", [(50, 0), (36, 0), (64, 0), (64, 1)])
@pytest.mark.parametrize("beta", [0.0, 0.5])
def test_output_pitch_and_untouched_padding(ldd, first, beta, tile):
    """D inside a padded buffer: pitches that do (36, 64) and do not (50) allow 16-byte
    row chunks, a D that starts off a 16-byte boundary (first column 1), and an N
    whose last chunk is partial; the padding must stay untouched."""
    M, N, K = 65, 33, 100
    A, B, C, alpha, _ = inputs(F16, F16, M, N, K, 9)
    Ad, Bd = to_dev_bits(A, F16), to_dev_bits(B, F16)
    buf = torch.full((M, ldd), 123.0, dtype=torch.float32, device=dev())
    Cd = torch.from_numpy(C).to(dev()) if beta != 0 else None
    with tile_shape(tile):
        mm.gemm_dense(Ad, Bd, buf[:, first:first + N], alpha, beta, Cd, a_type=F16, b_type=F16)
    torch.cuda.synchronize()
    out = buf.cpu().numpy()
    assert (out[:, :first] == 123.0).all() and (out[:, first + N:] == 123.0).all()
    Dref, S = oracle.gemm_dense(F16, F16, A, B, alpha, beta, C)
    assert_close(out[:, first:first + N], Dref, S, F16, K, alpha, beta, C)


@pytest.mark.parametrize("ta,tb", [(BF16, BF16), (E4M3, E5M2)])
def test_deterministic(ta, tb):
    M, N, K = 512, 512, 1024
    A, B, C, alpha, beta = inputs(ta, tb, M, N, K, 4)
    D1 = run_dense(ta, tb, A, B, alpha, beta, C)
    D2 = run_dense(ta, tb, A, B, alpha, beta, C)
    assert np.array_equal(D1, D2)


@pytest.mark.parametrize("ta,tb", PAIRS)
@pytest.mark.parametrize("M,N,K", [(1, 64, 64), (5, 100, 333), (16, 130, 1000), (17, 77, 200), (32, 300, 4100),
                                   (7, 40, 8192), (32, 33, 2176)])
def test_skinny_path_matches_oracle(ta, tb, M, N, K):
    """M <= 32 runs the skinny kernel (B streamed once, split K, fixed-order reduction).  The shapes
    cover K below one 128-byte chunk, a ragged last chunk, chunk counts below and far above the
    wave count (each wave's LDS ring wrapping many times), 32-row A and ragged N."""
    A, B, C, alpha, beta = inputs(ta, tb, M, N, K, M * 5 + N + K + ta + tb)
    with tile_shape(16):
        D = run_dense(ta, tb, A, B, alpha, beta, C)
    Dref, aux = oracle.gemm_dense(ta, tb, A, B, alpha, beta, C)
    if ta == I8:
        assert np.array_equal(D, Dref)
    else:
        assert_close(D, Dref, aux, ta, K, alpha, beta, C, f"skinny {ta},{tb} {M}x{N}x{K}")
    D2 = run_dense(ta, tb, A, B, alpha, beta, C)        # default choice, same kernel: same bits
    assert np.array_equal(D, D2)


@pytest.mark.parametrize("ta,alpha,beta", [(BF16, 1.0, 1.0), (BF16, 2.0, 0.5), (BF16, 0.0, 2.0), (E4M3, -1.0, 3.0),
                                            (I8, 1, 5), (I8, 1, -1), (I8, 0, 7), (I8, -2, 3)])
@pytest.mark.parametrize("tile", [256, 64])
def test_alpha_beta_combinations(ta, alpha, beta, tile):
    """beta * C is folded into the accumulator when alpha != 0 (floating) or alpha == 1 (int8),
    and applied in the epilogue otherwise; both must agree with the oracle."""
    tb = E5M2 if ta == E4M3 else ta
    M, N, K = 300, 270, 160
    A, B, C, _, _ = inputs(ta, tb, M, N, K, 31)
    with tile_shape(tile):
        D = run_dense(ta, tb, A, B, alpha, beta, C)
    Dref, aux = oracle.gemm_dense(ta, tb, A, B, alpha, beta, C)
    if ta == I8:
        assert np.array_equal(D, Dref)
    else:
        assert_close(D, Dref, aux, ta, K, alpha, beta, C, f"alpha {alpha} beta {beta}")


# (alpha, beta, A all zero): scale ratios far outside fp32 (2^+-200), a subnormal fp32 alpha, and
# equal extreme scales.  beta * C must keep its exact fp32 value whatever alpha is.
EXTREME_SCALES = [(2.0 ** -100, 2.0 ** 100, False), (2.0 ** 100, 2.0 ** -100, True), (1e-39, 1.0, False),
                  (2.0 ** -100, 2.0 ** -100, False), (1.0, 2.0 ** -120, False), (-3.0, 2.0 ** 60, False)]


@pytest.mark.parametrize("alpha,beta,a_zero", EXTREME_SCALES)
@pytest.mark.parametrize("tile", [256, 64])
@pytest.mark.parametrize("ta,tb", [(BF16, BF16), (E4M3, E5M2)])
def test_extreme_alpha_beta_ratios(ta, tb, alpha, beta, a_zero, tile):
    """alpha * A*B + beta * C for scales whose ratio leaves fp32's range.  The oracle gets alpha and
    beta as the fp32 values the library applies (the ABI rounds them once to fp32)."""
    M, N, K = 300, 270, 160
    A, B, C, _, _ = inputs(ta, tb, M, N, K, 37)
    if a_zero:
        A = np.zeros_like(A)
    with tile_shape(tile):
        D = run_dense(ta, tb, A, B, alpha, beta, C)
    a32, b32 = float(np.float32(alpha)), float(np.float32(beta))
    Dref, S = oracle.gemm_dense(ta, tb, A, B, a32, b32, C)
    assert np.isfinite(Dref).all()
    assert_close(D, Dref, S, ta, K, a32, b32, C, f"alpha {alpha} beta {beta}")
    if a_zero:                                    # D = beta * C exactly
        assert np.array_equal(D.astype(np.float64), Dref)
