"""Pins for the accumulator-layout formulas and the operation-count convention.

The forward and inverse formulas of every layout on the pages must compose to
the identity over their whole domain and reproduce the row-band tables the
pages print (tests/golden/acc_layout_rowbands.txt).  The per-instruction
operation counts the pages print (tests/golden/instruction_ops.txt) must all
equal 2*M*N*K*blocks, the convention the benchmark uses to count work.
"""
import os
import re

import pytest

from oracle import layouts as L

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rows_of(name):
    out = []
    for line in open(os.path.join(GOLDEN, name)):
        if line.strip() and not line.startswith("#"):
            out.append(line.split())
    return out


@pytest.mark.parametrize("shape,fwd,inv", [(32, L.fwd_32x32, L.inv_32x32),
                                           (16, L.fwd_16x16, L.inv_16x16),
                                           (4, L.fwd_4x4, L.inv_4x4)])
def test_dense_layout_is_a_bijection(shape, fwd, inv):
    blocks = L.blocks_of(shape)
    regs = L.regs_per_lane(shape, blocks)
    assert 64 * regs == blocks * shape * shape
    seen = set()
    for b in range(blocks):
        for i in range(shape):
            for j in range(shape):
                lane, reg = fwd(i, j, b)
                assert 0 <= lane < 64 and 0 <= reg < regs
                assert inv(lane, reg) == (i, j, b)
                seen.add((lane, reg))
    assert len(seen) == 64 * regs          # every (lane, reg) slot is used exactly once


@pytest.mark.parametrize("shape,fwd,inv", [(32, L.fwd_sparse_32x32, L.inv_sparse_32x32),
                                           (16, L.fwd_sparse_16x16, L.inv_sparse_16x16)])
def test_sparse_layout_is_one_block_of_dense(shape, fwd, inv):
    dense = {32: L.fwd_32x32, 16: L.fwd_16x16}[shape]
    slots = set()
    for i in range(shape):
        for j in range(shape):
            lane, reg = fwd(i, j)
            assert (lane, reg) == dense(i, j, 0)
            assert inv(lane, reg) == (i, j)
            slots.add((lane, reg))
    assert len(slots) == shape * shape and max(r for _, r in slots) + 1 == shape * shape // 64


def test_row_band_tables_match_formulas():
    fwd = {"dense32": L.fwd_32x32, "dense16": L.fwd_16x16,
           "sparse32": lambda i, j, b=0: L.fwd_sparse_32x32(i, j),
           "sparse16": lambda i, j, b=0: L.fwd_sparse_16x16(i, j)}
    shape = {"dense32": 32, "dense16": 16, "sparse32": 32, "sparse16": 16}
    covered = {k: set() for k in fwd}
    for name, r0, r1, l0, l1, g0, g1 in rows_of("acc_layout_rowbands.txt"):
        r0, r1, l0, l1, g0, g1 = map(int, (r0, r1, l0, l1, g0, g1))
        lanes, regs = set(), set()
        for i in range(r0, r1 + 1):
            covered[name].add(i)
            for j in range(shape[name]):
                lane, reg = fwd[name](i, j)
                lanes.add(lane)
                regs.add(reg)
        assert lanes == set(range(l0, l1 + 1)), (name, r0)
        if g0 >= 0:
            assert regs == set(range(g0, g1 + 1)), (name, r0)
    for name, rows in covered.items():
        assert rows == set(range(shape[name])), name


def test_block_one_adds_sixteen():
    for i in range(32):
        for j in range(32):
            (l0, g0), (l1, g1) = L.fwd_32x32(i, j, 0), L.fwd_32x32(i, j, 1)
            assert l0 == l1 and g1 == g0 + 16


NAME = re.compile(r"(s?mfmac?)_[fi]32_(\d+)x(\d+)x(\d+)")


def gemm_flops(M, N, K):
    """Work of one GEMM as the benchmark counts it: 2*M*N*K (dense-equivalent K for sparse A)."""
    import bench
    return bench.gemm_flops(M, N, K)


def test_instruction_ops_follow_two_mnk_blocks():
    rows = rows_of("instruction_ops.txt")
    assert len(rows) == 28
    for name, ops, cycles, coexec, elems in rows:
        fam, M, N, K = NAME.match(name).groups()
        M, N, K, ops, elems = int(M), int(N), int(K), int(ops), int(elems)
        if elems < 0:
            blocks = 1                       # sparse: block count 1, K is the dense K
        else:
            # M rows of A per lane group, 64/M lane groups, `elems` K values per lane
            # in each group: the groups hold 64/M * elems K values, i.e. that many
            # K values per block times the block count.
            assert (64 // M) * elems % K == 0
            blocks = (64 // M) * elems // K
        assert ops == 2 * M * N * K * blocks, name
        assert ops == gemm_flops(M, N, K) * blocks
        assert int(cycles) > int(coexec) >= 0


def test_page_block_count_rule_disagrees_for_doubled_k():
    """The dense page says packed-input variants have 64/M blocks regardless of K; its
    own operation counts contradict that for the doubled-K variants (one block)."""
    ops = {r[0]: int(r[1]) for r in rows_of("instruction_ops.txt")}
    assert ops["mfma_f32_32x32x8f16"] == 2 * 32 * 32 * 8 * 1 != 2 * 32 * 32 * 8 * (64 // 32)
    assert ops["mfma_f32_32x32x4f16"] == 2 * 32 * 32 * 4 * (64 // 32)
