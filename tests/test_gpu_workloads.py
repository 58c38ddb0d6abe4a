"""GPU parity at the full sizes of the benchmark workloads, in the launch configuration
the benchmark times (the library's default tile choice).

Small workloads are checked against the full oracle; the large ones against
oracle rows and entries that the CPU computes in seconds: two whole 256 x 256
output tiles (every wave, lane and register position of a workgroup) plus
random entries.  Compressor output is always compared in full, bit for bit.

Each large workload runs twice: with its own random inputs, against the
normwise and element-wise gates, and with exact inputs of the same shapes,
types, scales and sparsity structure (small integers, so that every fp32
partial sum is exact and the GPU must give the oracle's value bit for bit on
the sampled outputs; a lost K panel or a misplaced fragment cannot hide
there).
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_matrix_multiply_amd as mm
import workloads as W
from gpu_helpers import (SAMPLED_ENTRIES, assert_bits_equal, assert_close, compress_dev, dev, dev_bits_to_host,
                         out_tensor, sample_entries, to_dev_bits)

pytestmark = pytest.mark.gpu


def dense_on_gpu(w):
    Ad, Bd = to_dev_bits(w["A"], w["ta"]), to_dev_bits(w["B"], w["tb"])
    integer = w["ta"] == oracle.I8
    D = out_tensor(w["M"], w["N"], integer)
    Cd = torch.from_numpy(w["C"]).to(dev()) if w["beta"] != 0 else None
    mm.gemm_dense(Ad, Bd, D, w["alpha"], w["beta"], Cd, a_type=w["ta"], b_type=w["tb"])
    torch.cuda.synchronize()
    return D


def check_sampled(D, w, fn_entries, seed, exact=False):
    """The first and the last 256 x 256 output tile plus 65 536 random entries against the oracle:
    within the gates, or (exact inputs) bit for bit."""
    M, N, K = w["M"], w["N"], w["K"]
    ii, jj = sample_entries(M, N, SAMPLED_ENTRIES, seed, tiles=((0, 0), ((M - 1) // 256, (N - 1) // 256)))
    ref, S = fn_entries(ii, jj)
    got = D[torch.from_numpy(ii).to(dev()), torch.from_numpy(jj).to(dev())].cpu().numpy()
    if exact:
        return assert_bits_equal(got, ref, "sampled, exact inputs")
    C = w["C"][ii, jj] if w["beta"] != 0 else None
    return assert_close(got, ref, S, w["ta"], K, w["alpha"], w["beta"], C, "sampled")


def sparse_on_gpu(w):
    """The benchmark's sparse path: the GPU compresses A (checked in full against the oracle
    compressor, bit for bit), then the sparse GEMM runs on the GPU's own compressed operand."""
    ta, tb, M, N, K = w["ta"], w["tb"], w["M"], w["N"], w["K"]
    Ac_ref, idx_ref, bad_ref = oracle.compress24(ta, w["A"])
    Acd, idxd, bad = compress_dev(ta, to_dev_bits(w["A"], ta), M, K)
    torch.cuda.synchronize()
    assert int(bad.item()) == bad_ref
    assert np.array_equal(dev_bits_to_host(Acd, ta), Ac_ref)
    assert np.array_equal(idxd.cpu().numpy().view(np.uint32), idx_ref)
    D = out_tensor(M, N, False)
    mm.gemm_sparse24(Acd, idxd, to_dev_bits(w["B"], tb), D, K=K, alpha=w["alpha"], beta=w["beta"],
                     a_type=ta, b_type=tb)
    torch.cuda.synchronize()
    fn = lambda ii, jj: oracle.gemm_sparse24_entries(ta, tb, Ac_ref, idx_ref, w["B"], ii, jj, w["alpha"],
                                                     w["beta"], w["C"])
    return D, fn


@pytest.mark.parametrize("name", ["bf16_256", "i8_1024", "bf16_skinny"])
def test_small_workloads_full_oracle(name):
    w = W.workload(name)
    D = dense_on_gpu(w).cpu().numpy()
    Dref, aux = oracle.gemm_dense(w["ta"], w["tb"], w["A"], w["B"], w["alpha"], w["beta"], w["C"])
    if w["ta"] == oracle.I8:
        assert not aux                     # no int32 overflow in this workload
        assert np.array_equal(D, Dref)
    else:
        assert_close(D, Dref, aux, w["ta"], w["K"], w["alpha"], w["beta"], w["C"], name)


@pytest.mark.parametrize("name", ["bf16_4096", "bf16_8192", "fp8_8192"])
def test_large_dense_workloads_sampled(name):
    w = W.workload(name)
    D = dense_on_gpu(w)
    fn = lambda ii, jj: oracle.gemm_dense_entries(w["ta"], w["tb"], w["A"], w["B"], ii, jj, w["alpha"],
                                                  w["beta"], w["C"])
    check_sampled(D, w, fn, 7)


@pytest.mark.parametrize("name", ["bf16_4096_int", "bf16_8192_int", "fp8_8192_int"])
def test_large_dense_workloads_exact_inputs(name):
    w = W.workload(name)
    D = dense_on_gpu(w)
    fn = lambda ii, jj: oracle.gemm_dense_entries(w["ta"], w["tb"], w["A"], w["B"], ii, jj, w["alpha"],
                                                  w["beta"], w["C"])
    check_sampled(D, w, fn, 11, exact=True)


def test_skinny_workload_exact_inputs_full():
    w = W.workload("bf16_skinny_int")
    D = dense_on_gpu(w).cpu().numpy()
    Dref, _ = oracle.gemm_dense(w["ta"], w["tb"], w["A"], w["B"], w["alpha"], w["beta"], w["C"])
    assert_bits_equal(D, Dref, "skinny, exact inputs")


@pytest.mark.parametrize("name", ["f16_sparse", "fp8_8192_sparse"])
def test_sparse_workloads(name):
    w = W.workload(name)
    assert oracle.compress24(w["ta"], w["A"])[2] == 0
    D, fn = sparse_on_gpu(w)
    check_sampled(D, w, fn, 8)


@pytest.mark.parametrize("name", ["f16_sparse_int", "fp8_8192_int_sparse"])
def test_sparse_workloads_exact_inputs(name):
    w = W.workload(name)
    D, fn = sparse_on_gpu(w)
    check_sampled(D, w, fn, 12, exact=True)


def share_of(name, n_share=1024):
    """One GPU's share of an 8192^3 workload split 8 ways along N: all of A, the first
    n_share columns of B (and C)."""
    w = dict(W.workload(name))
    w["B"], w["N"] = np.ascontiguousarray(w["B"][:n_share]), n_share
    if w["C"] is not None:
        w["C"] = np.ascontiguousarray(w["C"][:, :n_share])
    return w


@pytest.mark.parametrize("name", ["bf16_8192", "fp8_8192"])
def test_share_shape_dense_sampled(name):
    w = share_of(name)
    D = dense_on_gpu(w)
    fn = lambda ii, jj: oracle.gemm_dense_entries(w["ta"], w["tb"], w["A"], w["B"], ii, jj, w["alpha"],
                                                  w["beta"], w["C"])
    check_sampled(D, w, fn, 9)


@pytest.mark.parametrize("name", ["bf16_8192_int", "fp8_8192_int"])
def test_share_shape_dense_exact_inputs(name):
    w = share_of(name)
    D = dense_on_gpu(w)
    fn = lambda ii, jj: oracle.gemm_dense_entries(w["ta"], w["tb"], w["A"], w["B"], ii, jj, w["alpha"],
                                                  w["beta"], w["C"])
    check_sampled(D, w, fn, 13, exact=True)


def test_share_shape_sparse_exact_inputs():
    w = share_of("fp8_8192_int_sparse")
    D, fn = sparse_on_gpu(w)
    check_sampled(D, w, fn, 14, exact=True)


def test_share_shape_sparse_sampled():
    w = share_of("fp8_8192_sparse")
    ta, tb, M, N, K = w["ta"], w["tb"], w["M"], w["N"], w["K"]
    Ac_ref, idx_ref, _ = oracle.compress24(ta, w["A"])
    Acd = to_dev_bits(Ac_ref, ta)
    idxd = torch.from_numpy(idx_ref.view(np.int32)).to(dev())
    D = out_tensor(M, N, False)
    mm.gemm_sparse24(Acd, idxd, to_dev_bits(w["B"], tb), D, K=K, alpha=w["alpha"], beta=w["beta"],
                     a_type=ta, b_type=tb)
    torch.cuda.synchronize()
    fn = lambda ii, jj: oracle.gemm_sparse24_entries(ta, tb, Ac_ref, idx_ref, w["B"], ii, jj, w["alpha"],
                                                     w["beta"], w["C"])
    check_sampled(D, w, fn, 10)
