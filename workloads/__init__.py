"""Seeded synthetic inputs for the GEMM workloads.

This module only draws random numbers and rounds them to the input formats
(with torch's round-to-nearest-even casts, fp8 after clamping to the largest
finite value).  It holds none of the GEMM or compression arithmetic; both the
GPU tests and the CPU oracle receive exactly the bytes produced here.

All arrays are numpy arrays of raw element bits (uint16 for fp16/bf16, int8
for int8, uint8 for fp8), A row-major M x K, B column-major K x N stored as an
N x K array, C row-major M x N (float32 or int32).

Seeds: seed = 20261200 + 10 * workload_id + operand (A=1, B=2, C=3, pattern=4).
"""
import numpy as np
import torch

F16, BF16, I8, E4M3, E5M2 = 1, 2, 3, 4, 5
_TORCH = {F16: torch.float16, BF16: torch.bfloat16, E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}
_BITS = {F16: np.uint16, BF16: np.uint16, E4M3: np.uint8, E5M2: np.uint8, I8: np.int8}
_FP8_MAX = {E4M3: 448.0, E5M2: 57344.0}


def seed_of(workload_id, operand):
    return 20261200 + 10 * int(workload_id) + {"A": 1, "B": 2, "C": 3, "pattern": 4}[operand]


def rng(workload_id, operand):
    return np.random.Generator(np.random.PCG64(seed_of(workload_id, operand)))


def to_bits(x, t):
    """Round float64 values to format t (saturating for fp8) and return the raw bits."""
    x = np.asarray(x, np.float64)
    if t in _FP8_MAX:
        x = np.clip(x, -_FP8_MAX[t], _FP8_MAX[t])
    y = torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).to(_TORCH[t])
    view = {2: torch.int16, 1: torch.uint8}[y.element_size()]
    return y.view(view).numpy().view(_BITS[t])


def from_bits(bits, t):
    """Raw bits -> float32 via torch's own cast (for building test fixtures only)."""
    bits = np.ascontiguousarray(bits)
    if t in (F16, BF16):
        return torch.from_numpy(bits.view(np.int16)).view(_TORCH[t]).to(torch.float32).numpy()
    return torch.from_numpy(bits.view(np.uint8)).view(_TORCH[t]).to(torch.float32).numpy()


def uniform(shape, t, workload_id, operand, lo=-1.0, hi=1.0):
    return to_bits(rng(workload_id, operand).uniform(lo, hi, size=shape), t)


def normal(shape, t, workload_id, operand, scale=1.0):
    return to_bits(rng(workload_id, operand).standard_normal(size=shape) * scale, t)


def int8_uniform(shape, workload_id, operand):
    return rng(workload_id, operand).integers(-128, 128, size=shape, dtype=np.int64).astype(np.int8)


def int32_uniform(shape, workload_id, operand, lo=-1000, hi=1000):
    return rng(workload_id, operand).integers(lo, hi + 1, size=shape, dtype=np.int64).astype(np.int32)


def float32_normal(shape, workload_id, operand):
    return rng(workload_id, operand).standard_normal(size=shape).astype(np.float32)


def small_int(shape, t, workload_id, operand, lo=-2, hi=2):
    """Integers drawn uniformly from [lo, hi], stored exactly in format t (fp16, bf16 and the
    fp8 formats hold every integer of magnitude <= 8 exactly).  Products of such inputs, and
    their sums while below 2^24, are exact in fp32 whatever the order of the additions."""
    x = rng(workload_id, operand).integers(lo, hi + 1, size=shape).astype(np.float64)
    return to_bits(x, t)


def int_valued_float32(shape, workload_id, operand, lo=-8, hi=8):
    return rng(workload_id, operand).integers(lo, hi + 1, size=shape).astype(np.float32)


# The six ways of keeping two of four positions, in the order the pattern draw uses.
PATTERNS = ((0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3))


def prune_mask(M, K, workload_id, patterns=None):
    """Boolean M x K keep-mask with exactly two kept positions in every group of four,
    one of the six patterns drawn uniformly per group (or taken from `patterns`,
    an M x K/4 array of indices into PATTERNS)."""
    assert K % 4 == 0
    if patterns is None:
        patterns = rng(workload_id, "pattern").integers(0, 6, size=(M, K // 4))
    table = np.zeros((6, 4), bool)
    for q, (a, b) in enumerate(PATTERNS):
        table[q, a] = table[q, b] = True
    return table[patterns].reshape(M, K)


def zero_bits(t):
    return np.zeros((), _BITS[t])


def sparse24_normal(M, K, t, workload_id, exact_two=True):
    """A ~ N(0,1) rounded to t, pruned to 4:2 with uniform patterns.
    exact_two=True redraws kept values that round to zero, so every group holds
    exactly two non-zeros; exact_two=False leaves them (random 2-of-4 pruning of
    a dense matrix)."""
    g = rng(workload_id, "A")
    x = g.standard_normal(size=(M, K))
    bits = to_bits(x, t)
    keep = prune_mask(M, K, workload_id)
    if exact_two:
        mag_mask = 0x7FFF if bits.dtype == np.uint16 else 0x7F
        while True:
            bad = keep & ((bits.astype(np.int64) & mag_mask) == 0)
            n = int(bad.sum())
            if n == 0:
                break
            bits[bad] = to_bits(g.standard_normal(size=n), t)
    bits = np.where(keep, bits, zero_bits(t))
    return np.ascontiguousarray(bits)


# ---- the workloads of the benchmark and the parity tests ---------------------

def workload(name):
    """Return a dict describing one named workload's inputs (host arrays of bits)."""
    if name == "bf16_256":       # dense bf16 256^3, U[-1,1), C = 0, alpha 1 beta 0
        M = N = K = 256
        return dict(ta=BF16, tb=BF16, M=M, N=N, K=K, alpha=1.0, beta=0.0,
                    A=uniform((M, K), BF16, 1, "A"), B=uniform((N, K), BF16, 1, "B"),
                    C=np.zeros((M, N), np.float32))
    if name == "i8_1024":        # dense int8 1024^3, C int32 U[-1000,1000], alpha = beta = 1
        M = N = K = 1024
        return dict(ta=I8, tb=I8, M=M, N=N, K=K, alpha=1, beta=1,
                    A=int8_uniform((M, K), 2, "A"), B=int8_uniform((N, K), 2, "B"),
                    C=int32_uniform((M, N), 2, "C"))
    if name in ("bf16_4096", "bf16_skinny", "bf16_8192"):
        M, N, K = {"bf16_4096": (4096, 4096, 4096), "bf16_skinny": (16, 4096, 4096),
                   "bf16_8192": (8192, 8192, 8192)}[name]
        wid = 3 if name != "bf16_8192" else 6
        s = 1.0 / np.sqrt(K)
        return dict(ta=BF16, tb=BF16, M=M, N=N, K=K, alpha=1.0, beta=1.0,
                    A=normal((M, K), BF16, wid, "A", s), B=normal((N, K), BF16, wid, "B", s),
                    C=float32_normal((M, N), wid, "C"))
    if name == "f16_sparse":     # 4:2 fp16, M = N = 4096, K = 8192, alpha 1 beta 0
        M, N, K = 4096, 4096, 8192
        return dict(ta=F16, tb=F16, M=M, N=N, K=K, alpha=1.0, beta=0.0,
                    A=sparse24_normal(M, K, F16, 4, exact_two=True),
                    B=normal((N, K), F16, 4, "B", 1.0 / np.sqrt(K)), C=None)
    if name in ("fp8_8192", "fp8_8192_sparse"):
        M = N = K = 8192
        A = normal((M, K), E4M3, 5, "A") if name == "fp8_8192" else sparse24_normal(M, K, E4M3, 5, False)
        return dict(ta=E4M3, tb=E5M2, M=M, N=N, K=K, alpha=1.0, beta=0.0,
                    A=A, B=normal((N, K), E5M2, 5, "B"), C=None)
    # Exact-input forms of the large workloads: the same shapes, types, alpha / beta and
    # sparsity structure, with small integers as values, so that every fp32 partial sum is an
    # exact integer (|sum| <= K * 4 + 8 < 2^24) and the GPU must equal the oracle bit for bit.
    if name in ("bf16_4096_int", "bf16_8192_int", "bf16_skinny_int"):
        M, N, K = {"bf16_4096_int": (4096, 4096, 4096), "bf16_8192_int": (8192, 8192, 8192),
                   "bf16_skinny_int": (16, 4096, 4096)}[name]
        wid = {"bf16_4096_int": 13, "bf16_8192_int": 16, "bf16_skinny_int": 17}[name]
        return dict(ta=BF16, tb=BF16, M=M, N=N, K=K, alpha=1.0, beta=1.0,
                    A=small_int((M, K), BF16, wid, "A"), B=small_int((N, K), BF16, wid, "B"),
                    C=int_valued_float32((M, N), wid, "C"))
    if name == "f16_sparse_int":
        M, N, K = 4096, 4096, 8192
        # kept values from {-2, -1, 1, 2}: exactly two non-zeros in every group
        keep = prune_mask(M, K, 14)
        mag = rng(14, "A").integers(1, 3, size=(M, K)) * rng(14, "C").choice([-1.0, 1.0], size=(M, K))
        A = np.where(keep, to_bits(mag, F16), zero_bits(F16))
        return dict(ta=F16, tb=F16, M=M, N=N, K=K, alpha=1.0, beta=0.0, A=np.ascontiguousarray(A),
                    B=small_int((N, K), F16, 14, "B"), C=None)
    if name in ("fp8_8192_int", "fp8_8192_int_sparse"):
        M = N = K = 8192
        A = small_int((M, K), E4M3, 15, "A")
        if name == "fp8_8192_int_sparse":      # random 2-of-4 pruning of the dense A (kept zeros stay)
            A = np.ascontiguousarray(np.where(prune_mask(M, K, 15), A, zero_bits(E4M3)))
        return dict(ta=E4M3, tb=E5M2, M=M, N=N, K=K, alpha=1.0, beta=0.0,
                    A=A, B=small_int((N, K), E5M2, 15, "B"), C=None)
    raise KeyError(name)
