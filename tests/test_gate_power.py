"""The floating parity gate can fail: on the CPU, with the oracle alone.

The pages' operation is an accumulation over K in panels, the caller looping
over K ("CDNA dense MFMA builtins", section "Naming convention"); the mistake
that loop invites is a lost panel.  Here the oracle computes, at the full
8192^3 workloads and on exactly the output positions the GPU parity tests
sample (two whole 256 x 256 tiles plus 65 536 random entries), both the true
result and the result of a kernel that skipped one k-tile -- every output
missing the same k-tile, or only the last output tile missing the last
k-tile.  The gate must accept the true result rounded to fp32 and reject
every planted loss.  No GPU is involved: the planted mistake is in the
oracle's input, never in a kernel.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import (SAMPLED_ENTRIES, elementwise_tolerance, gate_errors, gate_passes, sample_entries,
                         tolerance)

KTILE = {W.BF16: 64, W.E4M3: 128}      # dense K per k-tile of the tiled kernels


def _sampled(M, N, seed):
    return sample_entries(M, N, SAMPLED_ENTRIES, seed, tiles=((0, 0), ((M - 1) // 256, (N - 1) // 256)))


def _entries(w, A, ii, jj):
    return oracle.gemm_dense_entries(w["ta"], w["tb"], A, w["B"], ii, jj, w["alpha"], w["beta"], w["C"])


@pytest.mark.parametrize("name", ["bf16_8192", "fp8_8192"])
def test_gate_rejects_a_dropped_k_tile_at_8192(name):
    w = W.workload(name)
    M, N, K, t = w["M"], w["N"], w["K"], w["ta"]
    ii, jj = _sampled(M, N, 7)
    ref, S = _entries(w, w["A"], ii, jj)
    C = w["C"][ii, jj] if w["beta"] != 0 else None
    # the exact result rounded once to fp32 passes with a wide margin
    e, emax = gate_errors(ref.astype(np.float32), ref, S, w["alpha"], w["beta"], C)
    assert e <= tolerance(t, K) / 50 and emax <= elementwise_tolerance(t, K) / 50, (e, emax)

    kt = KTILE[t]
    for k0 in (0, K // 2, K - kt):                       # every output loses k-tile k0 / kt
        A = w["A"].copy()
        A[:, k0:k0 + kt] = 0
        bad, _ = _entries(w, A, ii, jj)
        e, emax = gate_errors(bad.astype(np.float32), ref, S, w["alpha"], w["beta"], C)
        assert e > 10 * tolerance(t, K), (k0, e)       # each gate alone rejects it
        assert emax > 3 * elementwise_tolerance(t, K), (k0, emax)

    # only the last 256 x 256 output tile loses the last k-tile
    A = w["A"].copy()
    A[:, K - kt:] = 0
    last = (ii >= (M - 1) // 256 * 256) & (jj >= (N - 1) // 256 * 256)
    bad_tile, _ = _entries(w, A, ii[last], jj[last])
    bad = ref.copy()
    bad[last] = bad_tile
    assert not gate_passes(bad.astype(np.float32), ref, S, t, K, w["alpha"], w["beta"], C)
    e, emax = gate_errors(bad.astype(np.float32), ref, S, w["alpha"], w["beta"], C)
    assert emax > 3 * elementwise_tolerance(t, K), emax


def test_gate_rejects_a_dropped_k_tile_sparse_fp8_8192():
    w = W.workload("fp8_8192_sparse")
    M, N, K, ta, tb = w["M"], w["N"], w["K"], w["ta"], w["tb"]
    Ac, idx, _ = oracle.compress24(ta, w["A"])
    ii, jj = _sampled(M, N, 8)
    ref, S = oracle.gemm_sparse24_entries(ta, tb, Ac, idx, w["B"], ii, jj)
    assert gate_passes(ref.astype(np.float32), ref, S, ta, K, 1.0, 0.0)
    kt = KTILE[ta]                                       # 128 dense K = 64 compressed values
    for k0 in (0, K // 2, K - kt):
        Acd = Ac.copy()
        Acd[:, k0 // 2:(k0 + kt) // 2] = 0
        bad, _ = oracle.gemm_sparse24_entries(ta, tb, Acd, idx, w["B"], ii, jj)
        e, emax = gate_errors(bad.astype(np.float32), ref, S, 1.0, 0.0)
        assert e > 10 * tolerance(ta, K), (k0, e)
        assert emax > 3 * elementwise_tolerance(ta, K), (k0, emax)


def test_gate_accepts_fp32_summation_in_any_order():
    """The gate's floor: a plain fp32 accumulation (in two different orders) of a random bf16
    product passes it; the element-wise bound holds for any order by construction."""
    rng = np.random.default_rng(3)
    M, N, K = 64, 48, 4096
    A = W.to_bits(rng.standard_normal((M, K)) / np.sqrt(K), W.BF16)
    B = W.to_bits(rng.standard_normal((N, K)) / np.sqrt(K), W.BF16)
    C = rng.standard_normal((M, N)).astype(np.float32)
    ref, S = oracle.gemm_dense(W.BF16, W.BF16, A, B, 1.0, 1.0, C)
    a = W.from_bits(A, W.BF16)
    b = W.from_bits(B, W.BF16)
    fwd = np.zeros((M, N), np.float32)
    for k in range(K):                                   # ascending k, fp32 adds
        fwd += np.outer(a[:, k], b[:, k]).astype(np.float32)
    rev = np.zeros((M, N), np.float32)
    for k in reversed(range(K)):                         # descending k
        rev += np.outer(a[:, k], b[:, k]).astype(np.float32)
    for acc in (fwd, rev):
        D = (acc + C).astype(np.float32)
        assert gate_passes(D, ref, S, W.BF16, K, 1.0, 1.0, C)
