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

# Gate of the floating parity tests: e = ||D - D_ref||_F / (|alpha| ||S||_F + |beta| ||C||_F)
# with S = sum_k |a*b|.  fp32 accumulation of K terms gives e of order 1e-7 * sqrt(K); the gates
# below are about 100x looser, and a layout or index mistake gives e of order 1.
def tolerance(t, K):
    return (1e-4 if t in FP8 else 1e-5) * np.sqrt(max(K, 1))


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
    e = oracle.normwise_error(D_gpu, D_ref, S, alpha, beta, C)
    tol = tolerance(t, K)
    assert np.isfinite(np.asarray(D_gpu)).all(), f"{what}: non-finite output"
    assert e <= tol, f"{what}: normwise error {e:.3e} > {tol:.3e}"
    return e


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
