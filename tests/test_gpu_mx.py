"""GPU parity of the block-scaled (MX) GEMM, mmac_gemm_dense_mx, against the oracle.

Every fp8/bf8 pair and tile shape, ragged M, N and K (K a multiple of 32 but not of the
128-element k-tile, so the last k-tile holds one to three blocks), scale exponents spread
over 2^-20 .. 2^20, garbage (255 included) in the scale bytes past K and in the pitch
padding, beta != 0, M <= 32; exact small-integer products with random power-of-two block
scales (bit for bit); the epilogue variants on top; and the 8192^3 fp8 x bf8 shape against
two whole 256 x 256 output tiles plus 65 536 sampled entries.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_matrix_multiply_amd as mm
import workloads as W
from gpu_helpers import (SAMPLED_ENTRIES, assert_close, dev, env, out_tensor, pack_mx_scales, sample_entries,
                         to_dev_bits)
from oracle import E4M3, E5M2

pytestmark = pytest.mark.gpu

PAIRS = [(E4M3, E4M3), (E4M3, E5M2), (E5M2, E4M3), (E5M2, E5M2)]


def mx_problem(ta, tb, M, N, K, seed, integers=False, lo=107, hi=148):
    g = np.random.default_rng(seed)
    if integers:
        A = W.to_bits(g.integers(-4, 5, size=(M, K)).astype(np.float64), ta)
        B = W.to_bits(g.integers(-4, 5, size=(N, K)).astype(np.float64), tb)
    else:
        A = W.to_bits(g.standard_normal((M, K)), ta)
        B = W.to_bits(g.standard_normal((N, K)), tb)
    SA = g.integers(lo, hi, size=(M, K // 32)).astype(np.uint8)
    SB = g.integers(lo, hi, size=(N, K // 32)).astype(np.uint8)
    C = g.standard_normal((M, N)).astype(np.float32)
    return A, B, SA, SB, C


def run_mx(ta, tb, A, SA, B, SB, alpha, beta, C, D=None, ld_pad=0, **kw):
    M, N = A.shape[0], B.shape[0]
    if D is None:
        D = out_tensor(M, N, False)
    SAd = pack_mx_scales(SA, ld=(M + 3) // 4 * 4 + ld_pad, seed=1)
    SBd = pack_mx_scales(SB, ld=(N + 3) // 4 * 4 + ld_pad, seed=2)
    Cd = torch.from_numpy(np.ascontiguousarray(C)).to(dev()) if beta != 0 and C is not None else None
    mm.gemm_mx(to_dev_bits(A, ta), SAd, to_dev_bits(B, tb), SBd, D, alpha, beta, Cd, a_type=ta, b_type=tb, **kw)
    torch.cuda.synchronize()
    return D


@pytest.mark.parametrize("ta,tb", PAIRS)
@pytest.mark.parametrize("tile", [256, 2561, 1282, 128, 64])
@pytest.mark.parametrize("M,N,K", [(64, 64, 128), (300, 260, 32 * 37), (33, 300, 1024), (257, 130, 96), (5, 7, 32)])
def test_mx_matches_oracle(ta, tb, tile, M, N, K):
    A, B, SA, SB, C = mx_problem(ta, tb, M, N, K, M + 3 * N + K + 7 * ta + tb)
    with env(MMAC_TILE=tile):
        D = run_mx(ta, tb, A, SA, B, SB, 1.25, -0.5, C, ld_pad=4).cpu().numpy()
    Dref, S = oracle.gemm_mx(ta, tb, A, SA, B, SB, 1.25, -0.5, C)
    assert_close(D, Dref, S, ta, K, 1.25, -0.5, C, f"mx {ta},{tb} {M}x{N}x{K} tile {tile}")


@pytest.mark.parametrize("ta,tb", PAIRS)
def test_mx_small_integers_exact(ta, tb):
    """|a|, |b| <= 4 with block exponents 2^-2 .. 2^2 on each side: every partial sum is a
    multiple of 2^-4 below 2^18, exact in fp32 -- the GPU must give the oracle's bits."""
    M, N, K = 130, 70, 32 * 21
    A, B, SA, SB, C = mx_problem(ta, tb, M, N, K, 5 + ta + tb, integers=True, lo=125, hi=130)
    C = np.round(C * 8) / 8
    for tile in (1282, 64):
        with env(MMAC_TILE=tile):
            D = run_mx(ta, tb, A, SA, B, SB, 1.0, 1.0, C).cpu().numpy()
        Dref, _ = oracle.gemm_mx(ta, tb, A, SA, B, SB, 1.0, 1.0, C)
        assert np.array_equal(D.astype(np.float64), Dref), f"tile {tile}"


def test_mx_epilogue_variant_exact():
    """bfloat16 C and D, bias and ReLU after the block-scaled sum (integer data, exact)."""
    ta, tb = E4M3, E5M2
    M, N, K = 200, 136, 512
    A, B, SA, SB, _ = mx_problem(ta, tb, M, N, K, 11, integers=True, lo=126, hi=129)
    g = np.random.default_rng(12)
    C = g.integers(-64, 65, size=(M, N)).astype(np.float32)
    bias = g.integers(-300, 301, size=N).astype(np.float32)
    Y, _ = oracle.gemm_mx(ta, tb, A, SA, B, SB, 1.0, 1.0, C)
    ref, _ = oracle.epilogue(Y, bias, mm.ACT_RELU, oracle.OUT_BF16)
    D = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev())
    Cd = torch.from_numpy(C).to(dev()).to(torch.bfloat16)
    mm.gemm_mx(to_dev_bits(A, ta), pack_mx_scales(SA), to_dev_bits(B, tb), pack_mx_scales(SB), D, 1.0, 1.0, Cd,
               a_type=ta, b_type=tb, bias=torch.from_numpy(bias).to(dev()), act=mm.ACT_RELU)
    torch.cuda.synchronize()
    assert np.array_equal(D.view(torch.int16).cpu().numpy().view(np.uint16), ref)


def test_mx_unit_scales_match_plain_fp8():
    """All exponents 127: the block-scaled GEMM is the plain fp8 GEMM (same tile shape, same
    summation order: the same bits)."""
    ta, tb = E4M3, E5M2
    M, N, K = 300, 270, 1024
    A, B, _, _, C = mx_problem(ta, tb, M, N, K, 13)
    ones_a = np.full((M, K // 32), 127, np.uint8)
    ones_b = np.full((N, K // 32), 127, np.uint8)
    with env(MMAC_TILE=1282):
        D = run_mx(ta, tb, A, ones_a, B, ones_b, 1.0, 0.0, None).cpu().numpy()
        D0 = out_tensor(M, N, False)
        mm.gemm_dense(to_dev_bits(A, ta), to_dev_bits(B, tb), D0, a_type=ta, b_type=tb)
        torch.cuda.synchronize()
    assert np.array_equal(D.view(np.uint32), D0.cpu().numpy().view(np.uint32))


def test_mx_8192_sampled():
    """The 8192^3 fp8 x bf8 workload's operands with random block exponents, in the launch
    configuration the library picks (128 x 256 tiles)."""
    w = W.workload("fp8_8192")
    ta, tb, M, N, K = w["ta"], w["tb"], w["M"], w["N"], w["K"]
    g = np.random.default_rng(31)
    SA = g.integers(117, 138, size=(M, K // 32)).astype(np.uint8)
    SB = g.integers(117, 138, size=(N, K // 32)).astype(np.uint8)
    D = run_mx(ta, tb, w["A"], SA, w["B"], SB, 1.0, 0.0, None)
    ii, jj = sample_entries(M, N, SAMPLED_ENTRIES, 14, tiles=((0, 0), ((M - 1) // 256, (N - 1) // 256)))
    ref, S = oracle.gemm_mx_entries(ta, tb, w["A"], SA, w["B"], SB, ii, jj)
    got = D[torch.from_numpy(ii).to(dev()), torch.from_numpy(jj).to(dev())].cpu().numpy()
    assert_close(got, ref, S, ta, K, 1.0, 0.0, None, "mx 8192^3")


# ----------------------------------------------------------------------- FP4 E2M1 --
FP4 = oracle.FP4


def fp4_problem(M, N, K, seed, lo=107, hi=148, small=False):
    g = np.random.default_rng(seed)
    if small:      # codes of magnitude <= 2 (0, 0.5, 1, 1.5, 2) and either sign
        mag = g.integers(0, 5, size=(M + N, K))
        sgn = g.integers(0, 2, size=(M + N, K)) << 3
        codes = (mag | sgn).astype(np.uint8)
    else:
        codes = g.integers(0, 16, size=(M + N, K)).astype(np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    A, B = packed[:M], packed[M:]
    SA = g.integers(lo, hi, size=(M, K // 32)).astype(np.uint8)
    SB = g.integers(lo, hi, size=(N, K // 32)).astype(np.uint8)
    return A, B, SA, SB


def run_fp4(A, SA, B, SB, alpha=1.0, beta=0.0, C=None, pad=0):
    M, N = A.shape[0], B.shape[0]
    def dev_packed(X):
        buf = torch.zeros((X.shape[0], X.shape[1] + pad), dtype=torch.uint8, device=dev())
        buf[:, :X.shape[1]] = torch.from_numpy(X).to(dev())
        return buf[:, :X.shape[1]]
    D = out_tensor(M, N, False)
    Cd = torch.from_numpy(np.ascontiguousarray(C)).to(dev()) if beta != 0 else None
    mm.gemm_mx(dev_packed(A), pack_mx_scales(SA, seed=3), dev_packed(B), pack_mx_scales(SB, seed=4), D, alpha, beta,
               Cd, a_type=FP4, b_type=FP4)
    torch.cuda.synchronize()
    return D


@pytest.mark.parametrize("tile", [256, 2561, 1282, 128, 64])
@pytest.mark.parametrize("M,N,K", [(64, 64, 256), (300, 260, 32 * 37), (33, 300, 1024), (257, 130, 96), (5, 7, 32)])
def test_mx_fp4_matches_oracle(tile, M, N, K):
    A, B, SA, SB = fp4_problem(M, N, K, M + N + K)
    C = np.random.default_rng(K).standard_normal((M, N)).astype(np.float32)
    with env(MMAC_TILE=tile):
        D = run_fp4(A, SA, B, SB, 0.75, 1.5, C, pad=16).cpu().numpy()
    Dref, S = oracle.gemm_mx(FP4, FP4, A, SA, B, SB, 0.75, 1.5, C)
    assert_close(D, Dref, S, E4M3, K, 0.75, 1.5, C, f"mx fp4 {M}x{N}x{K} tile {tile}")


def test_mx_fp4_exact():
    """|a|, |b| <= 2 with block exponents 2^-1 .. 2^1 on each side: multiples of 2^-4 below 2^16,
    exact in fp32 -- the oracle's bits."""
    M, N, K = 130, 70, 32 * 21
    A, B, SA, SB = fp4_problem(M, N, K, 3, lo=126, hi=129, small=True)
    for tile in (1282, 64):
        with env(MMAC_TILE=tile):
            D = run_fp4(A, SA, B, SB).cpu().numpy()
        Dref, _ = oracle.gemm_mx(FP4, FP4, A, SA, B, SB)
        assert np.array_equal(D.astype(np.float64), Dref), f"tile {tile}"


def test_mx_fp4_8192_sampled():
    M = N = K = 8192
    A, B, SA, SB = fp4_problem(M, N, K, 77, lo=117, hi=138)
    D = run_fp4(A, SA, B, SB)
    ii, jj = sample_entries(M, N, SAMPLED_ENTRIES, 15, tiles=((0, 0), ((M - 1) // 256, (N - 1) // 256)))
    ref, S = oracle.gemm_mx_entries(FP4, FP4, A, SA, B, SB, ii, jj)
    got = D[torch.from_numpy(ii).to(dev()), torch.from_numpy(jj).to(dev())].cpu().numpy()
    assert_close(got, ref, S, E4M3, K, 1.0, 0.0, None, "mx fp4 8192^3")


# ------------------------------------------------------------- FP6 E2M3 / BF6 E3M2 --
FP6, BF6 = oracle.FP6, oracle.BF6
FP6_PAIRS = [(FP6, FP6), (FP6, BF6), (BF6, FP6), (BF6, BF6)]


def pack6(codes):
    """rows x K six-bit codes -> rows x 3K/4 bytes, element n at bits 6n .. 6n+5 of the row."""
    bits = ((codes[:, :, None] >> np.arange(6)) & 1).astype(np.uint8).reshape(codes.shape[0], -1)
    return np.packbits(bits, axis=1, bitorder="little")


def fp6_problem(M, N, K, seed, lo=107, hi=148, small=False):
    g = np.random.default_rng(seed)
    if small:      # magnitudes <= 2 in either format (codes 0 .. 16) and either sign
        codes = g.integers(0, 17, size=(M + N, K)) | (g.integers(0, 2, size=(M + N, K)) << 5)
    else:
        codes = g.integers(0, 64, size=(M + N, K))
    packed = pack6(codes)
    SA = g.integers(lo, hi, size=(M, K // 32)).astype(np.uint8)
    SB = g.integers(lo, hi, size=(N, K // 32)).astype(np.uint8)
    return packed[:M], packed[M:], SA, SB


def run_fp6(ta, tb, A, SA, B, SB, alpha=1.0, beta=0.0, C=None, pad=0):
    M, N = A.shape[0], B.shape[0]

    def dev_packed(X):
        buf = torch.zeros((X.shape[0], X.shape[1] + pad), dtype=torch.uint8, device=dev())
        buf[:, :X.shape[1]] = torch.from_numpy(X).to(dev())
        return buf[:, :X.shape[1]]
    D = out_tensor(M, N, False)
    Cd = torch.from_numpy(np.ascontiguousarray(C)).to(dev()) if beta != 0 else None
    mm.gemm_mx(dev_packed(A), pack_mx_scales(SA, seed=5), dev_packed(B), pack_mx_scales(SB, seed=6), D, alpha, beta,
               Cd, a_type=ta, b_type=tb)
    torch.cuda.synchronize()
    return D


@pytest.mark.parametrize("ta,tb", FP6_PAIRS)
@pytest.mark.parametrize("tile", [2561, 1282, 128, 64])
@pytest.mark.parametrize("M,N,K", [(64, 64, 128), (300, 260, 32 * 37), (33, 300, 1024), (257, 130, 96), (5, 7, 32)])
def test_mx_fp6_matches_oracle(ta, tb, tile, M, N, K):
    """Rows of 3K/4 bytes padded to a 48-byte multiple of the pitch (lda a multiple of 64 elements)."""
    A, B, SA, SB = fp6_problem(M, N, K, M + N + K + 3 * ta + tb)
    pad = (-(K * 3 // 4)) % 48 + 48
    C = np.random.default_rng(K + 1).standard_normal((M, N)).astype(np.float32)
    with env(MMAC_TILE=tile):
        D = run_fp6(ta, tb, A, SA, B, SB, 0.75, 1.5, C, pad=pad).cpu().numpy()
    Dref, S = oracle.gemm_mx(ta, tb, A, SA, B, SB, 0.75, 1.5, C)
    assert_close(D, Dref, S, E4M3, K, 0.75, 1.5, C, f"mx fp6 {ta},{tb} {M}x{N}x{K} tile {tile}")


@pytest.mark.parametrize("ta,tb", FP6_PAIRS)
def test_mx_fp6_exact(ta, tb):
    """|a|, |b| <= 2 with block exponents 2^0 .. 2^1: multiples of 2^-8 below 2^14, exact in fp32 --
    the oracle's bits."""
    M, N, K = 130, 70, 32 * 21
    A, B, SA, SB = fp6_problem(M, N, K, 7 + ta + tb, lo=127, hi=129, small=True)
    pad = (-(K * 3 // 4)) % 48
    for tile in (1282, 64):
        with env(MMAC_TILE=tile):
            D = run_fp6(ta, tb, A, SA, B, SB, pad=pad).cpu().numpy()
        Dref, _ = oracle.gemm_mx(ta, tb, A, SA, B, SB)
        assert np.array_equal(D.astype(np.float64), Dref), f"tile {tile}"


def test_mx_fp6_8192_sampled():
    M = N = K = 8192
    A, B, SA, SB = fp6_problem(M, N, K, 78, lo=117, hi=138)
    D = run_fp6(FP6, BF6, A, SA, B, SB)
    ii, jj = sample_entries(M, N, SAMPLED_ENTRIES, 16, tiles=((0, 0), ((M - 1) // 256, (N - 1) // 256)))
    ref, S = oracle.gemm_mx_entries(FP6, BF6, A, SA, B, SB, ii, jj)
    got = D[torch.from_numpy(ii).to(dev()), torch.from_numpy(jj).to(dev())].cpu().numpy()
    assert_close(got, ref, S, E4M3, K, 1.0, 0.0, None, "mx fp6 8192^3")


@pytest.mark.parametrize("ta,tb", [(FP6, BF6), (FP4, FP4)])
def test_mx_packed_epilogue_variant_exact(ta, tb):
    """bfloat16 C and D, bias and ReLU after a packed FP6 / FP4 block-scaled sum (small values,
    power-of-two scales: exact)."""
    M, N, K = 200, 136, 512
    if ta == FP4:
        A, B, SA, SB = fp4_problem(M, N, K, 21, lo=126, hi=129, small=True)
    else:
        A, B, SA, SB = fp6_problem(M, N, K, 21, lo=127, hi=129, small=True)
    g = np.random.default_rng(22)
    C = g.integers(-64, 65, size=(M, N)).astype(np.float32)
    bias = g.integers(-300, 301, size=N).astype(np.float32)
    Y, _ = oracle.gemm_mx(ta, tb, A, SA, B, SB, 1.0, 1.0, C)
    ref, _ = oracle.epilogue(Y, bias, mm.ACT_RELU, oracle.OUT_BF16)
    D = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev())
    Cd = torch.from_numpy(C).to(dev()).to(torch.bfloat16)
    mm.gemm_mx(torch.from_numpy(A).to(dev()), pack_mx_scales(SA), torch.from_numpy(B).to(dev()), pack_mx_scales(SB),
               D, 1.0, 1.0, Cd, a_type=ta, b_type=tb, bias=torch.from_numpy(bias).to(dev()), act=mm.ACT_RELU)
    torch.cuda.synchronize()
    assert np.array_equal(D.view(torch.int16).cpu().numpy().view(np.uint16), ref)
