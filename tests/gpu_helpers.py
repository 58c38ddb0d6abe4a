"""Shared helpers of the GPU parity tests (host-side marshalling and comparison only)."""
import contextlib
import os

import numpy as np
import torch

import oracle
import sparse_matrix_multiply_amd as mm

# oracle type codes == library type codes
TORCH = {oracle.F16: torch.float16, oracle.BF16: torch.bfloat16, oracle.I8: torch.int8,
         oracle.E4M3: torch.float8_e4m3fn, oracle.E5M2: torch.float8_e5m2}
ESIZE = {oracle.F16: 2, oracle.BF16: 2, oracle.I8: 1, oracle.E4M3: 1, oracle.E5M2: 1}
FP8 = (oracle.E4M3, oracle.E5M2)

# Gates of the floating parity tests, with S = sum_k |a*b| and u = 2^-24 (fp32's unit roundoff).
# Every product of two inputs of these formats is exact in fp32, so with fp32 accumulation the only
# errors are the roundings of the sums and of the epilogue:
#   normwise:     e = ||D - D_ref||_F / (|alpha| ||S||_F + |beta| ||C||_F) <= 8 u sqrt(K)
#     (rounding errors of K random terms grow like sqrt(K); measured at 8192^3: 0.03-0.1 u sqrt(K));
#   element-wise: |D_ij - D_ref_ij| <= 2 (K + 2) u (|alpha| S_ij + |beta| |C_ij|)
#     (the worst case of K fp32 additions plus two epilogue roundings in any order, doubled so that
#     an accumulator that truncates instead of rounding also passes).
# The fp16 / bf16 instructions meet both everywhere.  The 8-, 6- and 4-bit instructions (the
# f8f6f4 MFMA and the fp8 SMFMAC) do not: measured on gfx950, one instruction's result carries an
# error of up to ~700 u of the S of its own K step at K = 64..128 (the sum inside an instruction is
# formed with fewer bits than fp32), so their gates add a bound per unit of S that does not grow
# with K:  normwise + 2^-15, element-wise + 2^-13 (about three times the largest error measured).
# A kernel that drops one k-tile of 64 (bf16) or 128 (fp8) K at 8192^3 still misses either gate by
# far (tests/test_gate_power.py shows it on the oracle).
U32 = 2.0 ** -24
NARROW = (oracle.E4M3, oracle.E5M2, oracle.FP4, oracle.FP6, oracle.BF6)   # instructions with narrow inner sums


def tolerance(t, K):
    return 8 * U32 * np.sqrt(max(K, 1)) + (2.0 ** -15 if t in NARROW else 0.0)


def elementwise_tolerance(t, K):
    return 2 * (max(K, 0) + 2) * U32 + (2.0 ** -13 if t in NARROW else 0.0)


def gate_errors(D_gpu, D_ref, S, alpha, beta, C=None):
    """(normwise e, largest element-wise ratio |D - D_ref| / (|alpha| S + |beta| |C|)); an element
    whose scale is zero must match exactly (ratio inf otherwise)."""
    D_gpu = np.asarray(D_gpu, np.float64)
    D_ref = np.asarray(D_ref, np.float64)
    e = oracle.normwise_error(D_gpu, D_ref, S, alpha, beta, C)
    scale = abs(alpha) * np.asarray(S, np.float64)
    if beta != 0 and C is not None:
        scale = scale + abs(beta) * np.abs(np.asarray(C, np.float64))
    diff = np.abs(D_gpu - D_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(scale > 0, diff / np.where(scale > 0, scale, 1.0), np.where(diff > 0, np.inf, 0.0))
    return e, (float(ratio.max()) if ratio.size else 0.0)


def gate_passes(D_gpu, D_ref, S, t, K, alpha, beta, C=None):
    e, emax = gate_errors(D_gpu, D_ref, S, alpha, beta, C)
    return e <= tolerance(t, K) and emax <= elementwise_tolerance(t, K)


def dev():
    return torch.device("cuda", 0)


def padded(n, t):
    """Smallest row pitch >= n whose byte size is a multiple of 16."""
    per = 16 // ESIZE[t]
    return max(per, (n + per - 1) // per * per)


def to_dev_bits(bits, t, ld=None):
    """Host array of raw bits (rows x cols) -> device tensor of type t with row pitch ld."""
    bits = np.ascontiguousarray(bits)
    rows, cols = bits.shape
    ld = padded(cols, t) if ld is None else ld
    if ESIZE[t] == 2:
        host = torch.from_numpy(bits.view(np.int16))
    else:
        host = torch.from_numpy(bits.view(np.int8))
    buf = torch.zeros((rows, ld), dtype=host.dtype, device=dev())
    buf[:, :cols] = host.to(dev())
    if t == oracle.I8:
        view = buf
    else:
        view = buf.view(TORCH[t])
    return view[:, :cols]


def dev_bits_to_host(x, t):
    """Device tensor of type t -> host numpy array of raw bits (same shape)."""
    y = x.contiguous()
    if ESIZE[t] == 2:
        return y.view(torch.int16).cpu().numpy().view(oracle.BITS_DTYPE[t])
    return y.view(torch.int8).cpu().numpy().view(oracle.BITS_DTYPE[t])


def out_tensor(M, N, integer, ld=None, fill=float("nan")):
    ld = N if ld is None else ld
    if integer:
        buf = torch.full((M, max(ld, 1)), -777, dtype=torch.int32, device=dev())
    else:
        buf = torch.full((M, max(ld, 1)), fill, dtype=torch.float32, device=dev())
    return buf[:, :N]


@contextlib.contextmanager
def env(**kv):
    """Set the library's tuning variables (read on every call) inside the block."""
    old = {k: os.environ.get(k) for k in kv}
    os.environ.update({k: str(v) for k, v in kv.items()})
    try:
        yield
    finally:
        for k, v in old.items():
            if v is None:
                del os.environ[k]
            else:
                os.environ[k] = v


def tile_shape(t):
    """Force the library's tile shape (MMAC_TILE) for the calls inside the block."""
    return env(MMAC_TILE=t)


def assert_close(D_gpu, D_ref, S, t, K, alpha, beta, C=None, what=""):
    assert np.isfinite(np.asarray(D_gpu)).all(), f"{what}: non-finite output"
    e, emax = gate_errors(D_gpu, D_ref, S, alpha, beta, C)
    tol, etol = tolerance(t, K), elementwise_tolerance(t, K)
    assert e <= tol, f"{what}: normwise error {e:.3e} > {tol:.3e}"
    assert emax <= etol, f"{what}: element-wise error {emax:.3e} > {etol:.3e}"
    return e


def assert_bits_equal(D_gpu, D_ref, what=""):
    """Exact-input checks: the fp32 output must equal the oracle's (exactly representable) value."""
    D_gpu = np.asarray(D_gpu)
    D_ref = np.asarray(D_ref, np.float64)
    assert np.array_equal(D_ref.astype(np.float32).astype(np.float64), D_ref), f"{what}: reference not exact in fp32"
    bad = np.flatnonzero(D_gpu.astype(np.float64) != D_ref)
    assert bad.size == 0, (f"{what}: {bad.size} of {D_ref.size} outputs differ; first at flat index {bad[0]}: "
                           f"{D_gpu.flat[bad[0]]!r} vs {D_ref.flat[bad[0]]!r}")


def run_dense(ta, tb, A, B, alpha, beta, C, ldd=None, C_dev=None):
    """Run mmac_gemm_dense on host inputs; returns D as a host array."""
    M, K = A.shape
    N = B.shape[0]
    Ad, Bd = to_dev_bits(A, ta), to_dev_bits(B, tb)
    integer = ta == oracle.I8
    if C_dev is None and C is not None:
        C_dev = torch.from_numpy(np.ascontiguousarray(C)).to(dev())
    D = out_tensor(M, N, integer, ldd)
    mm.gemm_dense(Ad, Bd, D, alpha, beta, C_dev if beta != 0 else None, a_type=ta, b_type=tb)
    torch.cuda.synchronize()
    return D.cpu().numpy()


def compress_dev(t, Ad, M, K, prune=False):
    """Run mmac_sparse24_compress (or, with prune, mmac_sparse24_prune_compress) on a device A;
    returns (Ac, idx, bad) device tensors."""
    Ac = to_dev_bits(np.zeros((M, K // 2), oracle.BITS_DTYPE[t]), t)
    W = (K + 31) // 32
    idx = torch.full((M, W), -1, dtype=torch.int32, device=dev())
    bad = torch.zeros(1, dtype=torch.int32, device=dev())
    (mm.sparse24_prune_compress if prune else mm.sparse24_compress)(Ad, Ac, idx, bad, a_type=t)
    return Ac, idx, bad


# Random output entries a full-size sampled check compares beside its whole tiles.
SAMPLED_ENTRIES = 65536


def sample_entries(M, N, n, seed, tiles=((0, 0),), tile=256):
    """Output positions for sampled checks: whole tile x tile blocks at the given tile
    coordinates (every lane / register / wave position) plus n random entries."""
    ii, jj = [], []
    for tr, tc in tiles:
        r0, c0 = tr * tile, tc * tile
        r = np.arange(r0, min(r0 + tile, M))
        c = np.arange(c0, min(c0 + tile, N))
        R, Cc = np.meshgrid(r, c, indexing="ij")
        ii.append(R.ravel())
        jj.append(Cc.ravel())
    g = np.random.default_rng(seed)
    ii.append(g.integers(0, M, n))
    jj.append(g.integers(0, N, n))
    return np.concatenate(ii).astype(np.int64), np.concatenate(jj).astype(np.int64)


def pack_mx_scales(S, ld=None, seed=0):
    """Row-major E8M0 exponents (rows x K/32 bytes) -> the library's scale-word layout:
    ceil(K/128) x ld int32 words, word (t, i) holding the exponents of blocks 4t .. 4t+3 of row i
    in bytes 0 .. 3.  The bytes of blocks past K/32 and the pitch padding are filled with random
    bytes (255 included): the library must ignore them."""
    S = np.ascontiguousarray(S, np.uint8)
    rows, nb = S.shape
    t = (nb + 3) // 4
    ld = ((rows + 3) // 4 * 4) if ld is None else ld
    g = np.random.default_rng(seed)
    full = g.integers(0, 256, size=(ld, 4 * t)).astype(np.uint8)
    full[:rows, :nb] = S
    words = full.view("<u4").reshape(ld, t).T                # (t, ld)
    return torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).to(dev())
