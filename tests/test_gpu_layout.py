"""GPU parity of mmac_gemm_dense_layout: A stored M-contiguous and / or B stored N-contiguous
(bf16 and fp16), the fragments of such an operand read from LDS with the transposing
ds_read_b64_tr_b16.  Every combination x every tile shape x ragged M, N and K (K tails
inside a k-tile), padded pitches, beta != 0; small-integer products bit for bit; an
epilogue variant; and the 8192^3 bf16 shape sampled."""
import numpy as np
import pytest
import torch

import oracle
import sparse_matrix_multiply_amd as mm
import workloads as W
from gpu_helpers import SAMPLED_ENTRIES, assert_close, dev, env, out_tensor, sample_entries
from oracle import BF16, F16

pytestmark = pytest.mark.gpu

LAYOUTS = [(True, False), (False, True), (True, True)]
TORCH = {BF16: torch.bfloat16, F16: torch.float16}


def dev16(bits, t, pad=8):
    """Host bits (rows x cols) -> device tensor of type t, row pitch padded to a multiple of 8."""
    rows, cols = bits.shape
    ld = (cols + 7) // 8 * 8 + pad
    buf = torch.zeros((rows, ld), dtype=torch.int16, device=dev())
    buf[:, :cols] = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev())
    return buf.view(TORCH[t])[:, :cols]


def run_layout(t, A, B, ta, tb, alpha, beta, C, D=None, **kw):
    """A (M x K) and B (N x K) host bits, stored on the device as asked."""
    M, N = A.shape[0], B.shape[0]
    Ad = dev16(np.ascontiguousarray(A.T) if ta else A, t)
    Bd = dev16(np.ascontiguousarray(B.T) if tb else B, t)
    D = out_tensor(M, N, False) if D is None else D
    Cd = torch.from_numpy(np.ascontiguousarray(C)).to(dev()) if beta != 0 else None
    mm.gemm_layout(Ad, Bd, D, ta, tb, alpha, beta, Cd, a_type=t, b_type=t, **kw)
    torch.cuda.synchronize()
    return D


@pytest.mark.parametrize("t", [BF16, F16])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("tile", [256, 2561, 1282, 128, 64])
@pytest.mark.parametrize("M,N,K", [(64, 64, 64), (300, 260, 333), (33, 300, 1000), (257, 130, 72), (5, 7, 9)])
def test_layout_matches_oracle(t, ta, tb, tile, M, N, K):
    g = np.random.default_rng(M + N + K + 10 * ta + 20 * tb + t)
    A = W.to_bits(g.standard_normal((M, K)), t)
    B = W.to_bits(g.standard_normal((N, K)), t)
    C = g.standard_normal((M, N)).astype(np.float32)
    with env(MMAC_TILE=tile):
        D = run_layout(t, A, B, ta, tb, 1.5, -0.5, C).cpu().numpy()
    Dref, S = oracle.gemm_dense(t, t, A, B, 1.5, -0.5, C)
    assert_close(D, Dref, S, t, K, 1.5, -0.5, C, f"layout {ta},{tb} {M}x{N}x{K} tile {tile}")


@pytest.mark.parametrize("t", [BF16, F16])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_layout_small_integers_exact(t, ta, tb):
    M, N, K = 130, 200, 520
    g = np.random.default_rng(5 + t)
    A = W.to_bits(g.integers(-4, 5, size=(M, K)).astype(np.float64), t)
    B = W.to_bits(g.integers(-4, 5, size=(N, K)).astype(np.float64), t)
    C = g.integers(-50, 51, size=(M, N)).astype(np.float32)
    Dref, _ = oracle.gemm_dense(t, t, A, B, 1.0, 1.0, C)
    for tile in (256, 64):
        with env(MMAC_TILE=tile):
            D = run_layout(t, A, B, ta, tb, 1.0, 1.0, C).cpu().numpy()
        assert np.array_equal(D.astype(np.float64), Dref), f"tile {tile}"


def test_layout_epilogue_variant():
    t = BF16
    M, N, K = 200, 136, 256
    g = np.random.default_rng(8)
    A = W.to_bits(g.integers(-4, 5, size=(M, K)).astype(np.float64), t)
    B = W.to_bits(g.integers(-4, 5, size=(N, K)).astype(np.float64), t)
    bias = g.integers(-300, 301, size=N).astype(np.float32)
    Y, _ = oracle.gemm_dense(t, t, A, B)
    ref, _ = oracle.epilogue(Y, bias, mm.ACT_RELU, oracle.OUT_BF16)
    D = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev())
    run_layout(t, A, B, True, True, 1.0, 0.0, None, D=D, bias=torch.from_numpy(bias).to(dev()), act=mm.ACT_RELU)
    assert np.array_equal(D.view(torch.int16).cpu().numpy().view(np.uint16), ref)


def test_layout_8192_sampled():
    """The 8192^3 bf16 workload (beta = 1) with B stored N-contiguous."""
    w = W.workload("bf16_8192")
    t, M, N, K = w["ta"], w["M"], w["N"], w["K"]
    D = run_layout(t, w["A"], w["B"], False, True, w["alpha"], w["beta"], w["C"])
    ii, jj = sample_entries(M, N, SAMPLED_ENTRIES, 16, tiles=((0, 0), ((M - 1) // 256, (N - 1) // 256)))
    ref, S = oracle.gemm_dense_entries(t, t, w["A"], w["B"], ii, jj, w["alpha"], w["beta"], w["C"])
    got = D[torch.from_numpy(ii).to(dev()), torch.from_numpy(jj).to(dev())].cpu().numpy()
    assert_close(got, ref, S, t, K, w["alpha"], w["beta"], w["C"][ii, jj], "layout 8192^3")


# ---------------------------------------------------------------- 8-bit elements --
# int8 and the four OCP fp8 / bf8 pairs; the transposed operand's fragments come through
# ds_read_b64_tr_b8.  int8 bit for bit (int32 wrap-around), fp8 within the fp8 gate.
from oracle import E4M3, E5M2, I8  # noqa: E402

PAIRS8 = [(I8, I8), (E4M3, E4M3), (E4M3, E5M2), (E5M2, E4M3), (E5M2, E5M2)]


def dev8(bits, pad=16):
    """Host bytes (rows x cols) -> device uint8 view with the row pitch padded to a multiple of 16."""
    rows, cols = bits.shape
    ld = (cols + 15) // 16 * 16 + pad
    buf = torch.zeros((rows, ld), dtype=torch.uint8, device=dev())
    buf[:, :cols] = torch.from_numpy(np.ascontiguousarray(bits).view(np.uint8)).to(dev())
    return buf[:, :cols]


def problem8(ta, tb, M, N, K, seed, small=False):
    g = np.random.default_rng(seed)
    if ta == I8:
        A = g.integers(-128, 128, size=(M, K)).astype(np.int8)
        B = g.integers(-128, 128, size=(N, K)).astype(np.int8)
        C = g.integers(-1000, 1001, size=(M, N)).astype(np.int32)
        return A, B, C, 3, -2
    draw = (lambda shape: g.integers(-4, 5, size=shape).astype(np.float64)) if small else g.standard_normal
    A = W.to_bits(draw((M, K)), ta)
    B = W.to_bits(draw((N, K)), tb)
    C = (np.round(g.standard_normal((M, N)) * 8) / 8 if small else g.standard_normal((M, N))).astype(np.float32)
    return A, B, C, (1.0 if small else 1.5), (1.0 if small else -0.5)


def run_layout8(ta, tb, A, B, trans_a, trans_b, alpha, beta, C, D=None):
    M, N = A.shape[0], B.shape[0]
    Ad = dev8(np.ascontiguousarray(A.T) if trans_a else A)
    Bd = dev8(np.ascontiguousarray(B.T) if trans_b else B)
    D = out_tensor(M, N, ta == I8) if D is None else D
    Cd = torch.from_numpy(np.ascontiguousarray(C)).to(dev()) if beta != 0 else None
    mm.gemm_layout(Ad, Bd, D, trans_a, trans_b, alpha, beta, Cd, a_type=ta, b_type=tb)
    torch.cuda.synchronize()
    return D


@pytest.mark.parametrize("ta,tb", PAIRS8)
@pytest.mark.parametrize("trans_a,trans_b", LAYOUTS)
@pytest.mark.parametrize("tile", [256, 2561, 1282, 128, 64])
@pytest.mark.parametrize("M,N,K", [(64, 64, 128), (300, 260, 333), (33, 300, 1000), (257, 130, 72)])
def test_layout8_matches_oracle(ta, tb, trans_a, trans_b, tile, M, N, K):
    A, B, C, alpha, beta = problem8(ta, tb, M, N, K, M + N + K + 10 * trans_a + 20 * trans_b + 3 * ta + tb)
    with env(MMAC_TILE=tile):
        D = run_layout8(ta, tb, A, B, trans_a, trans_b, alpha, beta, C).cpu().numpy()
    what = f"layout8 {ta},{tb} {trans_a},{trans_b} {M}x{N}x{K} tile {tile}"
    if ta == I8:
        Dref, _ = oracle.gemm_dense(ta, tb, A, B, alpha, beta, C)
        assert np.array_equal(D, Dref), what
    else:
        Dref, S = oracle.gemm_dense(ta, tb, A, B, alpha, beta, C)
        assert_close(D, Dref, S, ta, K, alpha, beta, C, what)


@pytest.mark.parametrize("ta,tb", PAIRS8[1:])
@pytest.mark.parametrize("trans_a,trans_b", LAYOUTS)
def test_layout8_small_integers_exact(ta, tb, trans_a, trans_b):
    """|a|, |b| <= 4: every partial sum is exact in fp32 -- the oracle's bits."""
    M, N, K = 130, 200, 520
    A, B, C, alpha, beta = problem8(ta, tb, M, N, K, 7 + ta + tb, small=True)
    Dref, _ = oracle.gemm_dense(ta, tb, A, B, alpha, beta, C)
    for tile in (256, 64):
        with env(MMAC_TILE=tile):
            D = run_layout8(ta, tb, A, B, trans_a, trans_b, alpha, beta, C).cpu().numpy()
        assert np.array_equal(D.astype(np.float64), Dref), f"tile {tile}"


def test_layout8_8192_sampled():
    """The 8192^3 fp8 x bf8 workload with A stored M-contiguous and B N-contiguous."""
    w = W.workload("fp8_8192")
    ta, tb, M, N, K = w["ta"], w["tb"], w["M"], w["N"], w["K"]
    D = run_layout8(ta, tb, w["A"], w["B"], True, True, 1.0, 0.0, None)
    ii, jj = sample_entries(M, N, SAMPLED_ENTRIES, 17, tiles=((0, 0), ((M - 1) // 256, (N - 1) // 256)))
    ref, S = oracle.gemm_dense_entries(ta, tb, w["A"], w["B"], ii, jj)
    got = D[torch.from_numpy(ii).to(dev()), torch.from_numpy(jj).to(dev())].cpu().numpy()
    assert_close(got, ref, S, ta, K, 1.0, 0.0, None, "layout8 8192^3")


@pytest.mark.parametrize("trans_a,trans_b", LAYOUTS)
def test_layout8_epilogue_variant(trans_a, trans_b):
    """fp8 x bf8 with transposed operands, bfloat16 D + bias + ReLU (integer products: exact)."""
    ta, tb = E4M3, E5M2
    M, N, K = 200, 136, 384
    A, B, _, _, _ = problem8(ta, tb, M, N, K, 31, small=True)
    g = np.random.default_rng(32)
    bias = g.integers(-300, 301, size=N).astype(np.float32)
    Y, _ = oracle.gemm_dense(ta, tb, A, B)
    ref, _ = oracle.epilogue(Y, bias, mm.ACT_RELU, oracle.OUT_BF16)
    D = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev())
    Ad = dev8(np.ascontiguousarray(A.T) if trans_a else A)
    Bd = dev8(np.ascontiguousarray(B.T) if trans_b else B)
    mm.gemm_layout(Ad, Bd, D, trans_a, trans_b, a_type=ta, b_type=tb, bias=torch.from_numpy(bias).to(dev()),
                   act=mm.ACT_RELU)
    torch.cuda.synchronize()
    assert np.array_equal(D.view(torch.int16).cpu().numpy().view(np.uint16), ref)
