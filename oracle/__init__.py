"""CPU oracle for the mmac GEMM library -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct implementation of what the GPU library
computes (dense and 4:2-sparse D = alpha*A*B + beta*C, and the 4:2
compressor), written in C (``mmac_oracle.c``) with fp64 / exact integer
accumulation and wrapped here with ctypes and numpy.  Only ``tests/``, the
smoke check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py``
may import this package.  It shares no code with the HIP library.

Arrays are numpy arrays of raw element bits: uint16 for fp16/bf16, int8 for
int8, uint8 for fp8 E4M3 / bf8 E5M2.  A is row-major M x K, B is column-major
K x N (passed as an N x K array), C and D are row-major M x N.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F16, BF16, I8, E4M3, E5M2, FP4, FP6, BF6 = 1, 2, 3, 4, 5, 6, 7, 8
FLOAT_TYPES = (F16, BF16, E4M3, E5M2)
BITS_DTYPE = {F16: np.uint16, BF16: np.uint16, I8: np.int8, E4M3: np.uint8, E5M2: np.uint8, FP4: np.uint8,
              FP6: np.uint8, BF6: np.uint8}
# FP4 (OCP E2M1) arrays are packed: rows x K/2 bytes, element 2m in the low nibble of byte m.
# FP6 (OCP E2M3 = FP6, E3M2 = BF6) arrays are packed: rows x 3K/4 bytes, element n of a row in
# bits 6n .. 6n+5 of the row read as a little-endian bit string.

_lib = None


def lib():
    """Load (building once if absent) the oracle's shared library."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        i64, dbl, vp, ip = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
        L.oracle_decode_one.restype = dbl
        L.oracle_decode_one.argtypes = [ip, ctypes.c_uint32]
        L.oracle_decode.argtypes = [ip, i64, vp, vp]
        L.oracle_gemm_dense_f64.argtypes = [ip, ip, i64, i64, i64, dbl, vp, i64, vp, i64, dbl, vp, i64,
                                            i64, i64, vp, i64, vp, i64]
        L.oracle_gemm_dense_f64_entries.argtypes = [ip, ip, i64, i64, i64, dbl, vp, i64, vp, i64, dbl, vp,
                                                    i64, i64, vp, vp, vp, vp]
        L.oracle_gemm_dense_i8.argtypes = [i64, i64, i64, i64, vp, i64, vp, i64, i64, vp, i64,
                                           i64, i64, vp, i64, vp]
        L.oracle_compress24.argtypes = [ip, i64, i64, vp, i64, vp, i64, vp, i64, vp]
        L.oracle_decompress24.argtypes = [ip, i64, i64, vp, i64, vp, i64, vp, i64]
        L.oracle_prune_compress24.argtypes = [ip, i64, i64, vp, i64, vp, i64, vp, i64, vp]
        L.oracle_epilogue.argtypes = [i64, i64, vp, i64, vp, ip, ip, vp, i64, vp]
        L.oracle_round.argtypes = [ip, i64, vp, vp]
        L.oracle_gemm_sparse24_f64.argtypes = [ip, ip, i64, i64, i64, dbl, vp, i64, vp, i64, vp, i64,
                                               dbl, vp, i64, i64, i64, vp, i64, vp, i64]
        L.oracle_gemm_sparse24_f64_entries.argtypes = [ip, ip, i64, i64, i64, dbl, vp, i64, vp, i64, vp,
                                                       i64, dbl, vp, i64, i64, vp, vp, vp, vp]
        L.oracle_gemm_sparse24_i8.argtypes = [i64, i64, i64, i64, vp, i64, vp, i64, vp, i64, i64, vp, i64,
                                              i64, i64, vp, i64, vp]
        L.oracle_gemm_mx_f64.argtypes = [ip, ip, i64, i64, i64, dbl, vp, i64, vp, i64, vp, i64, vp, i64, dbl, vp,
                                         i64, i64, i64, vp, i64, vp, i64]
        L.oracle_gemm_mx_f64_entries.argtypes = [ip, ip, i64, i64, i64, dbl, vp, i64, vp, i64, vp, i64, vp, i64,
                                                 dbl, vp, i64, i64, vp, vp, vp, vp]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        L.oracle_set_num_threads.restype = None
        _lib = L
    return _lib


def num_threads():
    """Threads the oracle's OpenMP loops use."""
    return int(lib().oracle_num_threads())


def set_num_threads(n):
    """Threads for later oracle calls (timing only: results do not depend on it)."""
    lib().oracle_set_num_threads(int(n))


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def _c2(a, dtype):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.dtype(dtype), (a.dtype, dtype)
    return a


def decode(t, bits):
    """Decode raw element bits of type t to float64 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=BITS_DTYPE[t])
    out = np.empty(bits.shape, np.float64)
    _check(lib().oracle_decode(t, bits.size, _p(bits), _p(out)), "decode")
    return out


def decode_one(t, bits):
    return lib().oracle_decode_one(t, int(bits))


def gemm_dense(ta, tb, A, B, alpha=1.0, beta=0.0, C=None, rows=None):
    """Dense GEMM.  Float types: returns (D fp64, S fp64) for output rows
    [r0, r1) (all rows by default), where S = sum_k |A*B| is the error scale.
    int8: returns (D int32 wrapped, out_of_range flag)."""
    M, K = A.shape
    N, K2 = B.shape
    assert K == K2
    r0, r1 = (0, M) if rows is None else rows
    if ta == I8:
        A, B = _c2(A, np.int8), _c2(B, np.int8)
        Cc = None if beta == 0 else _c2(C, np.int32)
        D = np.empty((r1 - r0, N), np.int32)
        oor = ctypes.c_int(0)
        _check(lib().oracle_gemm_dense_i8(M, N, K, int(alpha), _p(A), K, _p(B), K, int(beta), _p(Cc), N,
                                          r0, r1, _p(D), N, ctypes.byref(oor)), "gemm_dense_i8")
        return D, bool(oor.value)
    A, B = _c2(A, BITS_DTYPE[ta]), _c2(B, BITS_DTYPE[tb])
    Cc = None if beta == 0 else _c2(C, np.float32)
    D = np.empty((r1 - r0, N), np.float64)
    S = np.empty((r1 - r0, N), np.float64)
    _check(lib().oracle_gemm_dense_f64(ta, tb, M, N, K, float(alpha), _p(A), K, _p(B), K, float(beta),
                                       _p(Cc), N, r0, r1, _p(D), N, _p(S), N), "gemm_dense_f64")
    return D, S


def gemm_dense_entries(ta, tb, A, B, ii, jj, alpha=1.0, beta=0.0, C=None):
    """Dense floating GEMM at output positions (ii[q], jj[q]); returns (D, S) 1-D fp64."""
    M, K = A.shape
    N = B.shape[0]
    A, B = _c2(A, BITS_DTYPE[ta]), _c2(B, BITS_DTYPE[tb])
    Cc = None if beta == 0 else _c2(C, np.float32)
    ii = np.ascontiguousarray(ii, np.int64)
    jj = np.ascontiguousarray(jj, np.int64)
    out = np.empty(ii.shape, np.float64)
    S = np.empty(ii.shape, np.float64)
    _check(lib().oracle_gemm_dense_f64_entries(ta, tb, M, N, K, float(alpha), _p(A), K, _p(B), K,
                                               float(beta), _p(Cc), N, ii.size, _p(ii), _p(jj),
                                               _p(out), _p(S)), "gemm_dense_f64_entries")
    return out, S


def _mx_k(t, X):
    """Elements per row of an MX operand array (FP4 packs two per byte, FP6 four per three bytes)."""
    if t == FP4:
        return X.shape[1] * 2
    if t in (FP6, BF6):
        assert X.shape[1] % 3 == 0
        return X.shape[1] // 3 * 4
    return X.shape[1]


def gemm_mx(ta, tb, A, SA, B, SB, alpha=1.0, beta=0.0, C=None, rows=None):
    """Block-scaled (MX) GEMM: A M x K, B N x K (fp8 bits, packed FP4 bytes M x K/2 and N x K/2,
    or packed FP6 bytes M x 3K/4 and N x 3K/4), SA M x K/32 and SB N x K/32 E8M0 scale bytes; returns (D fp64, S fp64) for
    output rows [r0, r1)."""
    M, K = A.shape[0], _mx_k(ta, A)
    N = B.shape[0]
    assert _mx_k(tb, B) == K
    r0, r1 = (0, M) if rows is None else rows
    A, B = _c2(A, BITS_DTYPE[ta]), _c2(B, BITS_DTYPE[tb])
    SA, SB = _c2(SA, np.uint8), _c2(SB, np.uint8)
    assert SA.shape == (M, K // 32) and SB.shape == (N, K // 32)
    Cc = None if beta == 0 else _c2(C, np.float32)
    D = np.empty((r1 - r0, N), np.float64)
    S = np.empty((r1 - r0, N), np.float64)
    _check(lib().oracle_gemm_mx_f64(ta, tb, M, N, K, float(alpha), _p(A), K, _p(SA), K // 32, _p(B), K, _p(SB),
                                    K // 32, float(beta), _p(Cc), N, r0, r1, _p(D), N, _p(S), N), "gemm_mx_f64")
    return D, S


def gemm_mx_entries(ta, tb, A, SA, B, SB, ii, jj, alpha=1.0, beta=0.0, C=None):
    """Block-scaled GEMM at output positions (ii[q], jj[q]); returns (D, S) 1-D fp64."""
    M, K = A.shape[0], _mx_k(ta, A)
    N = B.shape[0]
    A, B = _c2(A, BITS_DTYPE[ta]), _c2(B, BITS_DTYPE[tb])
    SA, SB = _c2(SA, np.uint8), _c2(SB, np.uint8)
    Cc = None if beta == 0 else _c2(C, np.float32)
    ii = np.ascontiguousarray(ii, np.int64)
    jj = np.ascontiguousarray(jj, np.int64)
    out = np.empty(ii.shape, np.float64)
    S = np.empty(ii.shape, np.float64)
    _check(lib().oracle_gemm_mx_f64_entries(ta, tb, M, N, K, float(alpha), _p(A), K, _p(SA), K // 32, _p(B), K,
                                            _p(SB), K // 32, float(beta), _p(Cc), N, ii.size, _p(ii), _p(jj),
                                            _p(out), _p(S)), "gemm_mx_f64_entries")
    return out, S


def compress24(t, A):
    """Reference 4:2 compressor.  Returns (Ac M x K/2, idx M x ceil(K/32) uint32, bad_groups)."""
    A = _c2(A, BITS_DTYPE[t])
    M, K = A.shape
    Ac = np.zeros((M, K // 2), BITS_DTYPE[t])
    W = (K + 31) // 32
    idx = np.zeros((M, W), np.uint32)
    bad = ctypes.c_int64(0)
    _check(lib().oracle_compress24(t, M, K, _p(A), K, _p(Ac), K // 2, _p(idx), W, ctypes.byref(bad)),
           "compress24")
    return Ac, idx, int(bad.value)


def prune_compress24(t, A):
    """Magnitude pruning of a dense A to 4:2 (two largest |a| per group of four, NaN
    largest, ties to the lower position), then compression.  Returns
    (Ac, idx, groups_with_more_than_two_nonzeros)."""
    A = _c2(A, BITS_DTYPE[t])
    M, K = A.shape
    Ac = np.zeros((M, K // 2), BITS_DTYPE[t])
    W = (K + 31) // 32
    idx = np.zeros((M, W), np.uint32)
    bad = ctypes.c_int64(0)
    _check(lib().oracle_prune_compress24(t, M, K, _p(A), K, _p(Ac), K // 2, _p(idx), W, ctypes.byref(bad)),
           "prune_compress24")
    return Ac, idx, int(bad.value)


OUT_F32, OUT_BF16, OUT_F16, OUT_E4M3, OUT_E5M2 = 0, 1, 2, 3, 4
ACT_NONE, ACT_RELU = 0, 1


def epilogue(Y, bias=None, act=ACT_NONE, out_type=OUT_F32):
    """Epilogue variants on the exact GEMM value Y (float64 M x N): + bias[j] (float32),
    activation, rounding to the output format.  Returns (bits -- uint16 for bfloat16 /
    binary16, uint8 for E4M3 / E5M2 -- or a float32 array, the float64 value before rounding)."""
    Y = _c2(Y, np.float64)
    M, N = Y.shape
    dt = np.float32 if out_type == OUT_F32 else np.uint16 if out_type in (OUT_BF16, OUT_F16) else np.uint8
    out = np.zeros((M, N), dt)
    Yout = np.zeros((M, N), np.float64)
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    _check(lib().oracle_epilogue(M, N, _p(Y), N, _p(b) if b is not None else None, act, out_type, _p(out), N,
                                 _p(Yout)), "epilogue")
    return out, Yout


def round_to(out_type, x):
    """Round float64 values to bfloat16 (OUT_BF16), binary16 (OUT_F16) bits (uint16), or OCP
    E4M3 / E5M2 bits (uint8), saturating."""
    x = np.ascontiguousarray(x, np.float64)
    bits = np.zeros(x.shape, np.uint16)
    _check(lib().oracle_round(out_type, x.size, _p(x), _p(bits)), "round")
    return bits if out_type in (OUT_BF16, OUT_F16) else bits.astype(np.uint8)


def decompress24(t, Ac, idx, K):
    """Inverse of the compressor (positions not named by the index get +0)."""
    Ac = _c2(Ac, BITS_DTYPE[t])
    idx = _c2(idx, np.uint32)
    M = Ac.shape[0]
    A = np.zeros((M, K), BITS_DTYPE[t])
    _check(lib().oracle_decompress24(t, M, K, _p(Ac), Ac.shape[1], _p(idx), idx.shape[1], _p(A), K),
           "decompress24")
    return A


def gemm_sparse24(ta, tb, Ac, idx, B, alpha=1.0, beta=0.0, C=None, rows=None):
    """Sparse GEMM from the compressed form; same returns as gemm_dense."""
    M = Ac.shape[0]
    N, K = B.shape
    r0, r1 = (0, M) if rows is None else rows
    idx = _c2(idx, np.uint32)
    if ta == I8:
        Ac, B = _c2(Ac, np.int8), _c2(B, np.int8)
        Cc = None if beta == 0 else _c2(C, np.int32)
        D = np.empty((r1 - r0, N), np.int32)
        oor = ctypes.c_int(0)
        _check(lib().oracle_gemm_sparse24_i8(M, N, K, int(alpha), _p(Ac), Ac.shape[1], _p(idx), idx.shape[1],
                                             _p(B), K, int(beta), _p(Cc), N, r0, r1, _p(D), N,
                                             ctypes.byref(oor)), "gemm_sparse24_i8")
        return D, bool(oor.value)
    Ac, B = _c2(Ac, BITS_DTYPE[ta]), _c2(B, BITS_DTYPE[tb])
    Cc = None if beta == 0 else _c2(C, np.float32)
    D = np.empty((r1 - r0, N), np.float64)
    S = np.empty((r1 - r0, N), np.float64)
    _check(lib().oracle_gemm_sparse24_f64(ta, tb, M, N, K, float(alpha), _p(Ac), Ac.shape[1], _p(idx),
                                          idx.shape[1], _p(B), K, float(beta), _p(Cc), N, r0, r1,
                                          _p(D), N, _p(S), N), "gemm_sparse24_f64")
    return D, S


def gemm_sparse24_entries(ta, tb, Ac, idx, B, ii, jj, alpha=1.0, beta=0.0, C=None):
    """Sparse floating GEMM at output positions (ii[q], jj[q]); returns (D, S) 1-D fp64."""
    M = Ac.shape[0]
    N, K = B.shape
    Ac, B = _c2(Ac, BITS_DTYPE[ta]), _c2(B, BITS_DTYPE[tb])
    idx = _c2(idx, np.uint32)
    Cc = None if beta == 0 else _c2(C, np.float32)
    ii = np.ascontiguousarray(ii, np.int64)
    jj = np.ascontiguousarray(jj, np.int64)
    out = np.empty(ii.shape, np.float64)
    S = np.empty(ii.shape, np.float64)
    _check(lib().oracle_gemm_sparse24_f64_entries(ta, tb, M, N, K, float(alpha), _p(Ac), Ac.shape[1],
                                                  _p(idx), idx.shape[1], _p(B), K, float(beta), _p(Cc), N,
                                                  ii.size, _p(ii), _p(jj), _p(out), _p(S)),
           "gemm_sparse24_f64_entries")
    return out, S


def normwise_error(D_gpu, D_ref, S, alpha, beta, C=None):
    """e = ||D_gpu - D_ref||_F / (|alpha| ||S||_F + |beta| ||C||_F), the tests' gate metric."""
    diff = np.asarray(D_gpu, np.float64) - np.asarray(D_ref, np.float64)
    den = abs(alpha) * np.linalg.norm(S)
    if beta != 0 and C is not None:
        den += abs(beta) * np.linalg.norm(np.asarray(C, np.float64))
    num = np.linalg.norm(diff)
    if den == 0:
        return 0.0 if num == 0 else float("inf")
    return float(num / den)
