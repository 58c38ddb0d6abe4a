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
from gpu_helpers import assert_close, dev, env, out_tensor, sample_entries
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
    ii, jj = sample_entries(M, N, 20000, 16, tiles=((0, 0), ((M - 1) // 256, (N - 1) // 256)))
    ref, S = oracle.gemm_dense_entries(t, t, w["A"], w["B"], ii, jj, w["alpha"], w["beta"], w["C"])
    got = D[torch.from_numpy(ii).to(dev()), torch.from_numpy(jj).to(dev())].cpu().numpy()
    assert_close(got, ref, S, t, K, w["alpha"], w["beta"], w["C"][ii, jj], "layout 8192^3")
