"""Pins for the CPU oracle: each test checks it against something other than itself.

- decoders: every code of every format against torch's own casts, plus closed forms;
- dense GEMM: exact rational / integer brute force on small inputs, identity,
  permutation and one-hot products, beta = 0 ignoring a NaN C, int32 wrap-around;
- compressor: the index value the pages print for the {0,2} pattern, hand-worked
  groups, invariants over an exhaustive small alphabet, round trip;
- sparse GEMM: equal, bit for bit in fp64, to the dense GEMM on the decompressed A.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import BF16, E4M3, E5M2, F16, I8

TORCH = {F16: torch.float16, BF16: torch.bfloat16, E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}


def torch_decode(bits, t):
    """Decode raw bits with torch's casts (independent of the oracle's decoders)."""
    bits = np.ascontiguousarray(bits)
    if t == I8:
        return bits.astype(np.float64)
    if t in (F16, BF16):
        return torch.from_numpy(bits.view(np.int16)).view(TORCH[t]).to(torch.float64).numpy()
    return torch.from_numpy(bits.view(np.uint8)).view(TORCH[t]).to(torch.float64).numpy()


def same_values(a, b):
    a, b = np.asarray(a), np.asarray(b)
    nan_a, nan_b = np.isnan(a), np.isnan(b)
    assert np.array_equal(nan_a, nan_b)
    ok = ~nan_a
    assert np.array_equal(a[ok], b[ok])
    assert np.array_equal(np.signbit(a[ok]), np.signbit(b[ok]))


# ---------------------------------------------------------------- decoders --

@pytest.mark.parametrize("t,n", [(F16, 65536), (BF16, 65536), (E4M3, 256), (E5M2, 256)])
def test_decode_exhaustive_vs_torch(t, n):
    bits = np.arange(n, dtype=np.int64).astype(oracle.BITS_DTYPE[t])
    same_values(oracle.decode(t, bits), torch_decode(bits, t))


def test_decode_int8_exhaustive():
    bits = np.arange(-128, 128, dtype=np.int64).astype(np.int8)
    assert np.array_equal(oracle.decode(I8, bits), np.arange(-128, 128, dtype=np.float64))


def test_decode_closed_forms():
    d = oracle.decode_one
    assert d(E4M3, 0x7E) == 448.0 and d(E4M3, 0xFE) == -448.0     # largest finite E4M3
    assert d(E4M3, 0x01) == 2.0 ** -9                             # smallest subnormal
    assert np.isnan(d(E4M3, 0x7F)) and np.isnan(d(E4M3, 0xFF))    # S.1111.111 only NaN
    assert d(E4M3, 0x78) == 256.0                                 # exponent field 15 is finite
    assert d(E5M2, 0x7B) == 57344.0 and d(E5M2, 0x01) == 2.0 ** -16
    assert d(E5M2, 0x7C) == float("inf") and d(E5M2, 0xFC) == float("-inf")
    assert np.isnan(d(E5M2, 0x7D))
    assert d(F16, 0x7BFF) == 65504.0 and d(F16, 0x0001) == 2.0 ** -24 and d(F16, 0x3C00) == 1.0
    assert d(BF16, 0x3F80) == 1.0 and d(BF16, 0xC000) == -2.0 and d(BF16, 0x0001) == 2.0 ** -133
    assert d(I8, 0x80) == -128.0 and d(I8, 0x7F) == 127.0


# ------------------------------------------------------------- dense GEMM --

PAIRS = [(BF16, BF16), (F16, F16), (E4M3, E5M2), (E5M2, E4M3), (E4M3, E4M3), (E5M2, E5M2)]


def random_bits(shape, t, seed):
    g = np.random.default_rng(seed)
    if t == I8:
        return g.integers(-128, 128, size=shape).astype(np.int8)
    return W.to_bits(g.standard_normal(shape) * 2.0, t)


@pytest.mark.parametrize("ta,tb", PAIRS)
@pytest.mark.parametrize("M,N,K", [(4, 4, 4), (7, 5, 9), (32, 32, 32), (3, 17, 64)])
def test_dense_vs_exact_rational(ta, tb, M, N, K):
    seed = M * 1000 + N * 10 + K + 7 * ta + tb
    A, B = random_bits((M, K), ta, seed), random_bits((N, K), tb, seed + 1)
    C = np.random.default_rng(seed + 2).standard_normal((M, N)).astype(np.float32)
    alpha, beta = 0.75, -1.25
    D, S = oracle.gemm_dense(ta, tb, A, B, alpha, beta, C)
    Ad, Bd = torch_decode(A, ta), torch_decode(B, tb)
    for i in range(M):
        for j in range(N):
            exact = Fraction(0)
            for k in range(K):
                exact += Fraction(Ad[i, k]) * Fraction(Bd[j, k])
            exact = Fraction(alpha) * exact + Fraction(beta) * Fraction(float(C[i, j]))
            bound = (K + 3) * 2.0 ** -52 * (abs(alpha) * S[i, j] + abs(beta) * abs(float(C[i, j]))) + 1e-300
            assert abs(D[i, j] - float(exact)) <= bound, (i, j)
            assert S[i, j] == pytest.approx(float(sum(abs(Fraction(Ad[i, k]) * Fraction(Bd[j, k]))
                                                       for k in range(K))), rel=1e-12, abs=0)


@pytest.mark.parametrize("M,N,K", [(4, 4, 4), (9, 6, 33), (32, 32, 32)])
def test_dense_int8_vs_python_ints(M, N, K):
    A, B = random_bits((M, K), I8, M + K), random_bits((N, K), I8, N + K + 1)
    C = np.random.default_rng(3).integers(-1000, 1001, size=(M, N)).astype(np.int32)
    D, oor = oracle.gemm_dense(I8, I8, A, B, 3, -2, C)
    assert not oor
    for i in range(M):
        for j in range(N):
            v = 3 * sum(int(A[i, k]) * int(B[j, k]) for k in range(K)) - 2 * int(C[i, j])
            assert D[i, j] == v


def test_int8_wraps_mod_2_32():
    K = 64
    A = np.full((1, K), -128, np.int8)
    B = np.full((1, K), -128, np.int8)
    C = np.array([[2 ** 31 - 1]], np.int32)
    alpha, beta = 1000, 1
    exact = alpha * K * 128 * 128 + (2 ** 31 - 1)        # 1,048,576,000 + 2,147,483,647 > 2^31
    D, oor = oracle.gemm_dense(I8, I8, A, B, alpha, beta, C)
    assert oor
    wrapped = (exact + 2 ** 31) % 2 ** 32 - 2 ** 31
    assert int(D[0, 0]) == wrapped and wrapped < 0


@pytest.mark.parametrize("t", [BF16, F16, E4M3, E5M2])
def test_identity_permutation_onehot(t):
    n = 24
    one = W.to_bits(np.ones(1), t)[0]
    zero = W.zero_bits(t)
    B = random_bits((n, n), t, 11)             # B column-major: B[k, j] = Bst[j, k]
    Bd = torch_decode(B, t)
    # A = I  =>  D[i, j] = B[i, j] = Bst[j, i]
    A = np.full((n, n), zero, oracle.BITS_DTYPE[t])
    np.fill_diagonal(A, one)
    D, _ = oracle.gemm_dense(t, t, A, B)
    assert np.array_equal(D, Bd.T)
    # A = permutation P (row i picks column perm[i])  =>  D[i, :] = B[perm[i], :]
    perm = np.random.default_rng(5).permutation(n)
    P = np.full((n, n), zero, oracle.BITS_DTYPE[t])
    P[np.arange(n), perm] = one
    D, _ = oracle.gemm_dense(t, t, P, B)
    assert np.array_equal(D, Bd.T[perm, :])
    # one-hot A[2, 5] and B[5, 7] (i.e. Bst[7, 5])  =>  a single one at D[2, 7]
    A1 = np.full((n, n), zero, oracle.BITS_DTYPE[t]); A1[2, 5] = one
    B1 = np.full((n, n), zero, oracle.BITS_DTYPE[t]); B1[7, 5] = one
    D, _ = oracle.gemm_dense(t, t, A1, B1)
    expect = np.zeros((n, n)); expect[2, 7] = 1.0
    assert np.array_equal(D, expect)


def test_b_identity_and_alpha_beta():
    n = 16
    one, zero = W.to_bits(np.ones(1), BF16)[0], W.zero_bits(BF16)
    A = random_bits((n, n), BF16, 21)
    Bi = np.full((n, n), zero, np.uint16); np.fill_diagonal(Bi, one)
    C = np.random.default_rng(1).standard_normal((n, n)).astype(np.float32)
    D, _ = oracle.gemm_dense(BF16, BF16, A, Bi, 2.0, 0.5, C)
    assert np.array_equal(D, 2.0 * torch_decode(A, BF16) + 0.5 * C.astype(np.float64))


def test_beta_zero_ignores_nan_c():
    A, B = random_bits((8, 8), BF16, 1), random_bits((8, 8), BF16, 2)
    Cnan = np.full((8, 8), np.nan, np.float32)
    D0, _ = oracle.gemm_dense(BF16, BF16, A, B, 1.0, 0.0, None)
    D1, _ = oracle.gemm_dense(BF16, BF16, A, B, 1.0, 0.0, Cnan)
    assert np.isfinite(D1).all() and np.array_equal(D0, D1)


def test_row_ranges_and_entries_agree_with_full():
    A, B = random_bits((40, 48), E4M3, 3), random_bits((36, 48), E5M2, 4)
    C = np.random.default_rng(2).standard_normal((40, 36)).astype(np.float32)
    D, S = oracle.gemm_dense(E4M3, E5M2, A, B, 1.5, 0.5, C)
    Dr, Sr = oracle.gemm_dense(E4M3, E5M2, A, B, 1.5, 0.5, C, rows=(7, 19))
    assert np.array_equal(D[7:19], Dr) and np.array_equal(S[7:19], Sr)
    ii = np.array([0, 39, 13, 7]); jj = np.array([35, 0, 17, 7])
    De, Se = oracle.gemm_dense_entries(E4M3, E5M2, A, B, ii, jj, 1.5, 0.5, C)
    assert np.array_equal(De, D[ii, jj]) and np.array_equal(Se, S[ii, jj])


# ------------------------------------------------------------- compressor --

def test_index_value_printed_on_pages():
    """Keeping positions {0,2} of every group gives 0x88 for two groups and 0x8888 for four
    (the pages' fixed-pattern examples); a 32-wide span is then 0x88888888."""
    fixture = {}
    for line in open(__file__.replace("test_oracle_pins.py", "golden/sparsity_index.txt")):
        if line.strip() and not line.startswith("#"):
            g, v = line.split()
            fixture[int(g)] = int(v, 16)
    for t in (F16, E4M3):
        one = W.to_bits(np.ones(1), t)[0]
        for groups, value in fixture.items():
            K = 4 * groups
            A = np.full((3, K), W.zero_bits(t), oracle.BITS_DTYPE[t])
            A[:, 0::4] = one
            A[:, 2::4] = one
            Ac, idx, bad = oracle.compress24(t, A)
            assert bad == 0 and idx.shape == (3, 1)
            assert (idx[:, 0] == value).all()
            assert (Ac == one).all()
        A = np.full((2, 64), W.zero_bits(t), oracle.BITS_DTYPE[t])
        A[:, 0::4] = one
        A[:, 2::4] = one
        _, idx, _ = oracle.compress24(t, A)
        assert (idx == 0x88888888).all()


# hand-worked groups: (values as floats, expected kept positions, expected violation)
HAND = [
    ([0.0, 5.0, 0.0, 7.0], (1, 3), 0),
    ([2.0, 0.0, 0.0, -3.0], (0, 3), 0),
    ([0.0, 0.0, 1.5, 2.5], (2, 3), 0),
    ([4.0, 1.0, 0.0, 0.0], (0, 1), 0),
    ([0.0, 6.0, 8.0, 0.0], (1, 2), 0),
    ([0.0, 0.0, 0.0, 0.0], (0, 1), 0),       # no non-zero: pad with the two lowest
    ([0.0, 0.0, 0.0, 9.0], (0, 3), 0),       # one non-zero at 3: pad with 0
    ([0.0, 9.0, 0.0, 0.0], (0, 1), 0),       # one non-zero at 1: pad with 0
    ([0.0, 0.0, 9.0, 0.0], (0, 2), 0),
    ([1.0, 2.0, 3.0, 0.0], (0, 1), 1),       # three non-zeros: violation, keep lowest two
    ([1.0, 2.0, 3.0, 4.0], (0, 1), 1),
    ([0.0, 2.0, 3.0, 4.0], (1, 2), 1),
]
NIBBLE = {(0, 1): 0x4, (0, 2): 0x8, (0, 3): 0xC, (1, 2): 0x9, (1, 3): 0xD, (2, 3): 0xE}


@pytest.mark.parametrize("t", [F16, BF16, E4M3, E5M2])
def test_compress_hand_worked_groups(t):
    vals = np.array([v for g in HAND for v in g[0]])
    A = W.to_bits(vals, t).reshape(1, -1)
    Ac, idx, bad = oracle.compress24(t, A)
    assert bad == sum(g[2] for g in HAND)
    for g, (v, (p0, p1), _) in enumerate(HAND):
        nib = (int(idx[0, g // 8]) >> (4 * (g % 8))) & 0xF
        assert nib == NIBBLE[(p0, p1)], (g, v)
        assert Ac[0, 2 * g] == A[0, 4 * g + p0] and Ac[0, 2 * g + 1] == A[0, 4 * g + p1]


def test_compress_int8_minus128_is_nonzero():
    A = np.array([[0, -128, 0, 1]], np.int8)
    Ac, idx, bad = oracle.compress24(I8, A)
    assert bad == 0 and (int(idx[0, 0]) & 0xF) == NIBBLE[(1, 3)] and list(Ac[0]) == [-128, 1]


@pytest.mark.parametrize("t", [F16, E4M3])
def test_compress_exhaustive_small_alphabet(t):
    """All 625 groups over {+0, -0, 1, -1, NaN}: invariants of the compressor."""
    if t == F16:
        alphabet = [0x0000, 0x8000, 0x3C00, 0xBC00, 0x7E00]
    else:
        alphabet = [0x00, 0x80, 0x38, 0xB8, 0x7F]
    groups = list(itertools.product(range(5), repeat=4))
    A = np.array([[alphabet[s] for g in groups for s in g]], oracle.BITS_DTYPE[t])
    Ac, idx, bad = oracle.compress24(t, A)
    n_viol = 0
    for g, sym in enumerate(groups):
        nz = [p for p in range(4) if sym[p] not in (0, 1)]
        nib = (int(idx[0, g // 8]) >> (4 * (g % 8))) & 0xF
        p0, p1 = nib & 3, nib >> 2
        assert p0 < p1
        if len(nz) <= 2:
            assert set(nz) <= {p0, p1}          # every non-zero is kept
        else:
            n_viol += 1
            assert (p0, p1) == (nz[0], nz[1])   # the two lowest non-zeros
        assert Ac[0, 2 * g] == A[0, 4 * g + p0] and Ac[0, 2 * g + 1] == A[0, 4 * g + p1]
    assert bad == n_viol
    # the ragged index word: 625 groups -> 79 words, the last holds 1 group
    assert idx.shape == (1, 79) and (int(idx[0, 78]) >> 4) == 0


@pytest.mark.parametrize("t", [F16, BF16, E4M3, E5M2, I8])
def test_compress_matches_generator_pattern_and_round_trips(t):
    M, K = 13, 72                      # ragged: 72 = 2 full index words + 8 of 32
    pats = np.random.default_rng(9).integers(0, 6, size=(M, K // 4))
    keep = W.prune_mask(M, K, 0, patterns=pats)
    if t == I8:
        dense = np.random.default_rng(4).integers(1, 128, size=(M, K)).astype(np.int8)
        dense *= np.where(np.random.default_rng(5).random((M, K)) < 0.5, -1, 1).astype(np.int8)
        A = np.where(keep, dense, np.int8(0))
    else:
        dense = np.abs(np.random.default_rng(4).standard_normal((M, K))) + 0.5
        A = np.where(keep, W.to_bits(dense, t), W.zero_bits(t))
    Ac, idx, bad = oracle.compress24(t, A)
    assert bad == 0
    # compressed values are the kept ones in row order, nibbles name the drawn pattern
    assert np.array_equal(Ac, A[keep].reshape(M, K // 2))
    for i in range(M):
        for g in range(K // 4):
            nib = (int(idx[i, g // 8]) >> (4 * (g % 8))) & 0xF
            assert nib == NIBBLE[W.PATTERNS[pats[i, g]]]
    assert np.array_equal(oracle.decompress24(t, Ac, idx, K), A)


# ------------------------------------------------- magnitude prune + compress --
# Magnitude pruning is not on the pages (they give the 4:2 pattern and the
# compressed form only): keep the two largest |a| of each group of four, a NaN
# above every number, ties to the lower position.  Pinned by a rank-count
# brute force over torch-decoded values (a different algorithm from the
# oracle's sort), by hand-worked groups, and by agreement with the plain
# compressor wherever the input already has the 4:2 pattern.

def _mag_greater(x, y):
    if np.isnan(x) or np.isnan(y):
        return bool(np.isnan(x) and not np.isnan(y))
    return abs(x) > abs(y)


def _kept_by_rank(v):
    """Positions whose rank (elements ahead of them by magnitude, earlier position on ties) is < 2."""
    kept = []
    for p in range(4):
        ahead = sum(1 for q in range(4) if q != p and (_mag_greater(v[q], v[p]) or
                                                      (q < p and not _mag_greater(v[p], v[q]))))
        if ahead < 2:
            kept.append(p)
    return tuple(kept)


PRUNE_ALPHABET = {
    F16: [0x0000, 0x8000, 0x3C00, 0xBC00, 0x4000, 0xC000, 0x7C00, 0xFC00, 0x7E00, 0x0001],
    BF16: [0x0000, 0x8000, 0x3F80, 0xBF80, 0x4000, 0xC000, 0x7F80, 0xFF80, 0x7FC0, 0x0001],
    E4M3: [0x00, 0x80, 0x38, 0xB8, 0x40, 0xC0, 0x7E, 0xFE, 0x7F, 0x01],
    E5M2: [0x00, 0x80, 0x3C, 0xBC, 0x40, 0xC0, 0x7C, 0xFC, 0x7E, 0x01],
    I8: [0, 1, -1, 2, -2, 127, -127, -128, 64, -64],
}


@pytest.mark.parametrize("t", [F16, BF16, E4M3, E5M2, I8])
def test_prune_compress_vs_rank_brute_force(t):
    """Random groups over an alphabet with equal magnitudes, signed zeros, extremes, infinities
    and NaN (where the format has them), ragged K."""
    g = np.random.default_rng(31 + t)
    alpha = np.array(PRUNE_ALPHABET[t], oracle.BITS_DTYPE[t])
    M, K = 37, 4 * 75
    A = alpha[g.integers(0, len(alpha), size=(M, K))]
    Ac, idx, bad = oracle.prune_compress24(t, A)
    v = torch_decode(A, t)
    n_bad = 0
    for i in range(M):
        for gr in range(K // 4):
            grp = v[i, 4 * gr:4 * gr + 4]
            p0, p1 = _kept_by_rank(grp)
            nib = (int(idx[i, gr // 8]) >> (4 * (gr % 8))) & 0xF
            assert nib == NIBBLE[(p0, p1)], (i, gr, grp)
            assert Ac[i, 2 * gr] == A[i, 4 * gr + p0] and Ac[i, 2 * gr + 1] == A[i, 4 * gr + p1]
            n_bad += sum(1 for x in grp if x != 0 or np.isnan(x)) > 2
    assert bad == n_bad
    assert (int(idx[0, -1]) >> (4 * ((K // 4) % 8))) == 0    # bits past the last group stay clear


def test_prune_compress_hand_worked_groups():
    cases = [  # (type, group values, kept positions)
        (F16, [1.0, -3.0, 2.0, 0.5], (1, 2)),
        (F16, [1.0, 1.0, 1.0, 1.0], (0, 1)),
        (F16, [-1.0, 1.0, 2.0, -2.0], (2, 3)),
        (BF16, [0.25, -8.0, 0.0, 8.0], (1, 3)),
        (E4M3, [0.0, 0.0, -0.5, 0.0], (0, 2)),
        (E5M2, [float("nan"), 5.0, float("inf"), 1.0], (0, 2)),
        (E5M2, [1.0, float("-inf"), 2.0, 3.0], (1, 3)),
    ]
    for t, vals, (p0, p1) in cases:
        A = W.to_bits(np.array(vals), t).reshape(1, 4) if not any(np.isnan(vals)) else \
            np.array([[0x7E, 0x45, 0x7C, 0x3C]], np.uint8)          # E5M2 NaN, 5, inf, 1
        Ac, idx, bad = oracle.prune_compress24(t, A)
        assert int(idx[0, 0]) == NIBBLE[(p0, p1)], (t, vals)
        assert list(Ac[0]) == [A[0, p0], A[0, p1]]
    # signed zeros are copied bit for bit; -128 has the largest int8 magnitude
    A = np.array([[0x8000, 0x0000, 0x0000, 0x8000]], np.uint16)
    Ac, idx, _ = oracle.prune_compress24(F16, A)
    assert int(idx[0, 0]) == NIBBLE[(0, 1)] and list(Ac[0]) == [0x8000, 0x0000]
    A = np.array([[127, -128, 0, -127]], np.int8)
    Ac, idx, bad = oracle.prune_compress24(I8, A)
    assert int(idx[0, 0]) == NIBBLE[(0, 1)] and list(Ac[0]) == [127, -128] and bad == 1


@pytest.mark.parametrize("t", [F16, BF16, E4M3, E5M2, I8])
def test_prune_compress_equals_compress_on_4_2_input(t):
    """Where every group already has at most two non-zeros, pruning changes nothing."""
    M, K = 11, 4 * 41
    pats = np.random.default_rng(12).integers(0, 6, size=(M, K // 4))
    keep = W.prune_mask(M, K, 0, patterns=pats) & (np.random.default_rng(13).random((M, K)) > 0.15)
    if t == I8:
        dense = np.random.default_rng(14).integers(-128, 128, size=(M, K)).astype(np.int8)
        A = np.where(keep, dense, np.int8(0))
    else:
        A = np.where(keep, W.to_bits(np.random.default_rng(14).standard_normal((M, K)), t), W.zero_bits(t))
    got, want = oracle.prune_compress24(t, A), oracle.compress24(t, A)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1]) and got[2] == want[2] == 0


# ------------------------------------------------------------ sparse GEMM --

@pytest.mark.parametrize("ta,tb", [(F16, F16), (BF16, BF16), (E4M3, E5M2), (E5M2, E5M2)])
def test_sparse_equals_dense_on_decompressed(ta, tb):
    M, N, K = 19, 23, 136
    A = W.sparse24_normal(M, K, ta, 77, exact_two=False)
    A[0, :8] = W.to_bits(np.array([1, 2, 3, 0, 0, 0, 0, 0.0]), ta)   # one violating group
    B = random_bits((N, K), tb, 5)
    C = np.random.default_rng(8).standard_normal((M, N)).astype(np.float32)
    Ac, idx, bad = oracle.compress24(ta, A)
    assert bad == 1
    Ad = oracle.decompress24(ta, Ac, idx, K)       # the 4:2 matrix the sparse path sees
    Ds, Ss = oracle.gemm_sparse24(ta, tb, Ac, idx, B, 1.25, -0.5, C)
    Dd, Sd = oracle.gemm_dense(ta, tb, Ad, B, 1.25, -0.5, C)
    assert np.array_equal(Ds, Dd) and np.array_equal(Ss, Sd)
    ii = np.array([0, 18, 5]); jj = np.array([22, 0, 11])
    De, Se = oracle.gemm_sparse24_entries(ta, tb, Ac, idx, B, ii, jj, 1.25, -0.5, C)
    assert np.array_equal(De, Ds[ii, jj]) and np.array_equal(Se, Ss[ii, jj])


def test_sparse_int8_equals_dense_on_decompressed():
    M, N, K = 11, 9, 96
    pats = np.random.default_rng(1).integers(0, 6, size=(M, K // 4))
    keep = W.prune_mask(M, K, 0, patterns=pats)
    A = np.where(keep, random_bits((M, K), I8, 2), np.int8(0))
    B = random_bits((N, K), I8, 3)
    C = np.random.default_rng(4).integers(-1000, 1001, size=(M, N)).astype(np.int32)
    Ac, idx, _ = oracle.compress24(I8, A)
    Ds, o1 = oracle.gemm_sparse24(I8, I8, Ac, idx, B, 2, 3, C)
    Dd, o2 = oracle.gemm_dense(I8, I8, oracle.decompress24(I8, Ac, idx, K), B, 2, 3, C)
    assert np.array_equal(Ds, Dd) and o1 == o2


def test_sparse_rejects_invalid_nibble():
    Ac = np.zeros((1, 2), np.uint16)
    idx = np.array([[0x5]], np.uint32)          # p0 = 1, p1 = 1: not a pair
    B = np.zeros((1, 4), np.uint16)
    with pytest.raises(ValueError):
        oracle.gemm_sparse24(F16, F16, Ac, idx, B)


def test_normwise_error_metric():
    D = np.array([[1.0, 2.0]]); S = np.array([[3.0, 4.0]])
    assert oracle.normwise_error(D + np.array([[0.0, 0.5]]), D, S, 1.0, 0.0) == pytest.approx(0.1)


# -------------------------------------------------------- output epilogue --
# Rounding to bfloat16 / binary16 (nearest, ties to even, saturating) and the
# bias + ReLU step are not on the pages; they are pinned by round trips over
# every code, by torch's own float64 casts, and by hand-worked ties.

@pytest.mark.parametrize("out_type,t", [(oracle.OUT_BF16, BF16), (oracle.OUT_F16, F16)])
def test_round_trips_every_code(out_type, t):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = torch_decode(codes, t)
    back = oracle.round_to(out_type, vals)
    finite_or_inf = ~np.isnan(vals)
    assert np.array_equal(back[finite_or_inf], codes[finite_or_inf])
    nan_code = 0x7FC0 if t == BF16 else 0x7E00
    assert np.all((back[~finite_or_inf] & 0x7FFF) == nan_code)


@pytest.mark.parametrize("out_type,tdt,maxf", [(oracle.OUT_BF16, torch.bfloat16, 3.3895313892515355e38),
                                               (oracle.OUT_F16, torch.float16, 65504.0)])
def test_rounding_matches_torch_in_range_and_saturates(out_type, tdt, maxf):
    g = np.random.default_rng(17)
    x = np.concatenate([g.standard_normal(20000) * np.exp(g.uniform(-40, 40, 20000)),
                        g.uniform(-1e-7, 1e-7, 2000), g.uniform(-maxf, maxf, 2000)])
    # values exact in float32: torch converts float64 through float32 (a second rounding)
    x = x.astype(np.float32).astype(np.float64)
    ours = oracle.round_to(out_type, x)
    theirs = torch.from_numpy(x).to(tdt).view(torch.int16).numpy().astype(np.uint16)
    over = np.isinf(torch.from_numpy(x).to(tdt).float().numpy())
    assert np.array_equal(ours[~over], theirs[~over])
    # beyond the largest finite value: saturated, sign kept
    sat = oracle.round_to(out_type, np.array([maxf * 2, -maxf * 2, np.inf, -np.inf]))
    top = 0x7F7F if out_type == oracle.OUT_BF16 else 0x7BFF
    inf = 0x7F80 if out_type == oracle.OUT_BF16 else 0x7C00
    assert list(sat) == [top, top | 0x8000, inf, inf | 0x8000]


def test_rounding_ties_to_even():
    f16 = oracle.round_to(oracle.OUT_F16, np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, -(1 + 2 ** -11), 2 ** -25,
                                                    3 * 2 ** -25]))
    assert list(f16) == [0x3C00, 0x3C02, 0xBC00, 0x0000, 0x0002]
    bf16 = oracle.round_to(oracle.OUT_BF16, np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 2 ** -134, 3 * 2 ** -134]))
    assert list(bf16) == [0x3F80, 0x3F82, 0x0000, 0x0002]


def test_epilogue_bias_and_relu():
    Y = np.array([[1.5, -2.0, 0.0], [np.nan, -0.25, 3.0]])
    bias = np.array([0.25, 1.0, -4.0], np.float32)
    out, y = oracle.epilogue(Y, bias, oracle.ACT_RELU, oracle.OUT_F32)
    assert np.array_equal(out[0], np.array([1.75, 0.0, 0.0], np.float32))
    assert np.isnan(out[1, 0]) and out[1, 1] == 0.75 and out[1, 2] == 0.0
    out, _ = oracle.epilogue(Y, None, oracle.ACT_NONE, oracle.OUT_BF16)
    assert list(out[0]) == [0x3FC0, 0xC000, 0x0000]


# OCP fp8 output (E4M3 / E5M2): every code round-trips, torch's casts agree in range,
# hand-worked ties and the saturation rules (E4M3 has no infinity: it saturates too).
@pytest.mark.parametrize("out_type,t", [(oracle.OUT_E4M3, E4M3), (oracle.OUT_E5M2, E5M2)])
def test_fp8_round_trips_every_code(out_type, t):
    codes = np.arange(256, dtype=np.uint8)
    vals = torch_decode(codes, t)
    back = oracle.round_to(out_type, vals)
    nan = np.isnan(vals)
    assert np.array_equal(back[~nan], codes[~nan])
    assert np.all((back[nan] & 0x7F) == (0x7F if t == E4M3 else 0x7E))


@pytest.mark.parametrize("out_type,tdt,maxf", [(oracle.OUT_E4M3, torch.float8_e4m3fn, 448.0),
                                               (oracle.OUT_E5M2, torch.float8_e5m2, 57344.0)])
def test_fp8_rounding_matches_torch_in_range(out_type, tdt, maxf):
    g = np.random.default_rng(23)
    x = np.concatenate([g.uniform(-maxf, maxf, 20000), g.standard_normal(20000) * np.exp(g.uniform(-20, 5, 20000))])
    x = x.astype(np.float32).astype(np.float64)          # one rounding on both sides
    x = x[np.abs(x) <= maxf]
    ours = oracle.round_to(out_type, x)
    theirs = torch.from_numpy(x.astype(np.float32)).to(tdt).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_fp8_ties_and_saturation():
    e4 = oracle.round_to(oracle.OUT_E4M3, np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 464.0, 465.0, 1e30,
                                                    np.inf, -np.inf, np.nan, -0.0]))
    assert list(e4) == [0x38, 0x3A, 0x00, 0x02, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7F, 0x80]
    e5 = oracle.round_to(oracle.OUT_E5M2, np.array([1.125, 1.375, 2.0 ** -17, 3 * 2.0 ** -17, 61440.0, 1e30,
                                                    np.inf, -np.inf, np.nan]))
    assert list(e5) == [0x3C, 0x3E, 0x00, 0x02, 0x7B, 0x7B, 0x7C, 0xFC, 0x7E]
    out, _ = oracle.epilogue(np.array([[3.0, -500.0]]), np.array([0.25, 0.0], np.float32), oracle.ACT_NONE,
                             oracle.OUT_E4M3)
    assert out.dtype == np.uint8 and list(out[0]) == [0x45, 0xFE]      # 3.25 -> 3.25 (0x45), -500 -> -448


# ------------------------------------------------------ block-scaled (MX) GEMM --
# Not on the pages: the OCP microscaling definition (blocks of 32 along K, one
# E8M0 scale 2^(e - 127) per block of a row of A and of a column of B).

MX_PAIRS = [(E4M3, E4M3), (E4M3, E5M2), (E5M2, E4M3), (E5M2, E5M2)]


def mx_inputs(ta, tb, M, N, K, seed, lo=117, hi=138):
    g = np.random.default_rng(seed)
    A = W.to_bits(g.standard_normal((M, K)), ta)
    B = W.to_bits(g.standard_normal((N, K)), tb)
    SA = g.integers(lo, hi, size=(M, K // 32)).astype(np.uint8)
    SB = g.integers(lo, hi, size=(N, K // 32)).astype(np.uint8)
    return A, B, SA, SB


@pytest.mark.parametrize("ta,tb", MX_PAIRS)
def test_mx_brute_force_fraction(ta, tb):
    """Exact rational brute force (torch-decoded values, scales as Fractions)."""
    M, N, K = 5, 4, 64
    A, B, SA, SB = mx_inputs(ta, tb, M, N, K, ta * 10 + tb)
    C = np.random.default_rng(1).standard_normal((M, N)).astype(np.float32)
    D, S = oracle.gemm_mx(ta, tb, A, SA, B, SB, 0.75, -1.5, C)
    Av, Bv = torch_decode(A, ta), torch_decode(B, tb)
    for i in range(M):
        for j in range(N):
            acc = Fraction(0)
            for k in range(K):
                sc = Fraction(2) ** (int(SA[i, k // 32]) - 127) * Fraction(2) ** (int(SB[j, k // 32]) - 127)
                acc += sc * Fraction(Av[i, k]) * Fraction(Bv[j, k])
            want = Fraction(0.75) * acc + Fraction(-1.5) * Fraction(float(C[i, j]))
            assert D[i, j] == float(want)


@pytest.mark.parametrize("ta,tb", MX_PAIRS)
def test_mx_unit_scales_equal_dense(ta, tb):
    M, N, K = 9, 7, 96
    A, B, _, _ = mx_inputs(ta, tb, M, N, K, 3)
    ones_a = np.full((M, K // 32), 127, np.uint8)
    ones_b = np.full((N, K // 32), 127, np.uint8)
    D, S = oracle.gemm_mx(ta, tb, A, ones_a, B, ones_b)
    D0, S0 = oracle.gemm_dense(ta, tb, A, B)
    assert np.array_equal(D, D0) and np.array_equal(S, S0)


def test_mx_block_scales_act_per_block():
    """Raising one block's exponent by d multiplies exactly that block's contribution by 2^d;
    the scale of a block of A acts on its row, that of B on its column; 255 is NaN."""
    ta = tb = E4M3
    M, N, K = 3, 2, 96
    A, B, SA, SB = mx_inputs(ta, tb, M, N, K, 9, 127, 128)       # all scales 127
    parts = []
    for b in range(3):
        keep = np.zeros((1, K), bool)
        keep[0, 32 * b:32 * b + 32] = True
        Ab = np.where(keep, A, W.zero_bits(ta)).astype(A.dtype)
        parts.append(oracle.gemm_mx(ta, tb, Ab, SA, B, SB)[0])
    SA2 = SA.copy()
    SA2[1, 2] += 3
    SB2 = SB.copy()
    SB2[0, 0] -= 2
    D, _ = oracle.gemm_mx(ta, tb, A, SA2, B, SB2)
    want = parts[0] + parts[1] + parts[2]
    want[1, :] += 7 * parts[2][1, :]                   # block 2 of row 1: x 2^3
    want[:, 0] -= 0.75 * parts[0][:, 0]                # block 0 of column 0: x 2^-2
    assert np.allclose(D, want, rtol=0, atol=1e-12)
    SA2[2, 1] = 255
    D, _ = oracle.gemm_mx(ta, tb, A, SA2, B, SB2)
    assert np.isnan(D[2]).all() and np.isfinite(D[:2]).all()


def test_mx_entries_match_full():
    ta, tb = E5M2, E4M3
    M, N, K = 40, 30, 128
    A, B, SA, SB = mx_inputs(ta, tb, M, N, K, 4)
    C = np.random.default_rng(2).standard_normal((M, N)).astype(np.float32)
    D, S = oracle.gemm_mx(ta, tb, A, SA, B, SB, 1.5, 0.5, C)
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    De, Se = oracle.gemm_mx_entries(ta, tb, A, SA, B, SB, ii.ravel(), jj.ravel(), 1.5, 0.5, C)
    assert np.array_equal(De, D.ravel()) and np.array_equal(Se, S.ravel())


# FP4 (OCP E2M1, two per byte, element 2m in the low nibble of byte m) for block-scaled GEMMs.
FP4_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]          # codes 0..7; 8..15 are their negatives


def fp4_unpack(P):
    P = np.asarray(P, np.uint8)
    lo, hi = P & 15, P >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(P.shape[0], -1)
    mag = np.array(FP4_VALUES)[codes & 7]
    return np.where(codes & 8, -mag, mag)


def test_fp4_decode_every_code():
    got = [oracle.decode_one(oracle.FP4, c) for c in range(16)]
    want = FP4_VALUES + [-v for v in FP4_VALUES]
    assert got == want and np.signbit(got[8])


def test_mx_fp4_brute_force_fraction():
    g = np.random.default_rng(41)
    M, N, K = 4, 3, 64
    A = g.integers(0, 256, size=(M, K // 2)).astype(np.uint8)
    B = g.integers(0, 256, size=(N, K // 2)).astype(np.uint8)
    SA = g.integers(120, 135, size=(M, K // 32)).astype(np.uint8)
    SB = g.integers(120, 135, size=(N, K // 32)).astype(np.uint8)
    D, S = oracle.gemm_mx(oracle.FP4, oracle.FP4, A, SA, B, SB, 2.0, 0.0)
    Av, Bv = fp4_unpack(A), fp4_unpack(B)
    for i in range(M):
        for j in range(N):
            acc = sum(Fraction(2) ** (int(SA[i, k // 32]) + int(SB[j, k // 32]) - 254) * Fraction(Av[i, k]) *
                      Fraction(Bv[j, k]) for k in range(K))
            assert D[i, j] == float(2 * acc)
            assert S[i, j] == float(sum(abs(Fraction(2) ** (int(SA[i, k // 32]) + int(SB[j, k // 32]) - 254) *
                                            Fraction(Av[i, k]) * Fraction(Bv[j, k])) for k in range(K)))


# FP6 (OCP E2M3 and E3M2, four elements in three bytes: element n of a row in bits 6n .. 6n+5 of
# the row read as a little-endian bit string) for block-scaled GEMMs.  Each format's 32 non-negative
# codes run through its binades in order: subnormals, then equal steps inside each power of two.
# The OCP microscaling specification fixes the end points checked here: E2M3 max 7.5, smallest
# normal 1, smallest subnormal 1/8; E3M2 max 28, smallest normal 1/4, smallest subnormal 1/16.
FP6_VALUES = np.concatenate([np.arange(0, 1, 1 / 8), np.arange(1, 2, 1 / 8), np.arange(2, 4, 1 / 4),
                             np.arange(4, 8, 1 / 2)]).tolist()
BF6_VALUES = np.concatenate([np.arange(0, 1 / 4, 1 / 16), np.arange(1 / 4, 1 / 2, 1 / 16),
                             np.arange(1 / 2, 1, 1 / 8), np.arange(1, 2, 1 / 4), np.arange(2, 4, 1 / 2),
                             np.arange(4, 8, 1), np.arange(8, 16, 2), np.arange(16, 32, 4)]).tolist()


def fp6_unpack(P, t):
    """Packed FP6 rows -> values, through numpy's own little-endian bit unpacking."""
    P = np.asarray(P, np.uint8)
    bits = np.unpackbits(P, axis=1, bitorder="little")                  # rows x 8 * bytes
    codes = (bits.reshape(P.shape[0], -1, 6) * (1 << np.arange(6))).sum(axis=2)
    table = np.array(FP6_VALUES if t == oracle.FP6 else BF6_VALUES)
    mag = table[codes & 31]
    return np.where(codes & 32, -mag, mag)


@pytest.mark.parametrize("t,table,top,norm,sub", [(oracle.FP6, FP6_VALUES, 7.5, 1.0, 0.125),
                                                 (oracle.BF6, BF6_VALUES, 28.0, 0.25, 0.0625)])
def test_fp6_decode_every_code(t, table, top, norm, sub):
    assert len(table) == 32 and table[-1] == top and table[1] == sub
    mbits = 3 if t == oracle.FP6 else 2
    assert table[1 << mbits] == norm                      # first code with a non-zero exponent field
    got = [oracle.decode_one(t, c) for c in range(64)]
    assert got == table + [-v for v in table] and np.signbit(got[32])


@pytest.mark.parametrize("ta,tb", [(oracle.FP6, oracle.FP6), (oracle.FP6, oracle.BF6), (oracle.BF6, oracle.FP6),
                                   (oracle.BF6, oracle.BF6)])
def test_mx_fp6_brute_force_fraction(ta, tb):
    g = np.random.default_rng(43 + 2 * ta + tb)
    M, N, K = 4, 3, 96
    A = g.integers(0, 256, size=(M, K * 3 // 4)).astype(np.uint8)
    B = g.integers(0, 256, size=(N, K * 3 // 4)).astype(np.uint8)
    SA = g.integers(120, 135, size=(M, K // 32)).astype(np.uint8)
    SB = g.integers(120, 135, size=(N, K // 32)).astype(np.uint8)
    C = g.standard_normal((M, N)).astype(np.float32)
    D, S = oracle.gemm_mx(ta, tb, A, SA, B, SB, 0.5, 1.25, C)
    Av, Bv = fp6_unpack(A, ta), fp6_unpack(B, tb)
    assert Av.shape == (M, K)
    for i in range(M):
        for j in range(N):
            terms = [Fraction(2) ** (int(SA[i, k // 32]) + int(SB[j, k // 32]) - 254) * Fraction(Av[i, k]) *
                     Fraction(Bv[j, k]) for k in range(K)]
            assert D[i, j] == float(Fraction(1, 2) * sum(terms) + Fraction(5, 4) * Fraction(float(C[i, j])))
            assert S[i, j] == float(sum(abs(t) for t in terms))


def test_mx_fp6_element_position():
    """One non-zero code at element n of a packed row of A lands on k = n alone: against a B whose
    column j holds 1 at k = j only, D[0][j] is non-zero exactly for j = n (every n of a 64-element row)."""
    K = 64
    one = 0b001000                                          # E2M3: exponent field 1, mantissa 0 -> 1.0
    B = np.zeros((K, K * 3 // 4), np.uint8)
    for j in range(K):                                      # column j of B: 1.0 at element j
        bit = 6 * j
        v = one << (bit % 8)
        B[j, bit // 8] |= v & 255
        if v >> 8:
            B[j, bit // 8 + 1] |= v >> 8
    ones = np.full((K, 2), 127, np.uint8)
    for n in range(K):
        A = B[n:n + 1].copy()
        D, _ = oracle.gemm_mx(oracle.FP6, oracle.FP6, A, ones[:1], B, ones)
        assert np.nonzero(D[0])[0].tolist() == [n] and D[0, n] == 1.0
