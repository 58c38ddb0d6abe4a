"""Python binding of libmmac: tiled dense and 4:2-sparse GEMM for MI355X (gfx950).

Thin ctypes layer over the C ABI in include/mmac.h, with the same entry
points.  It only marshals arguments: torch tensors provide device memory and
the current HIP stream; every step of the computation runs in the library's
HIP kernels.  If libmmac.so is missing, importing the binding succeeds but the
first call raises -- there is no fallback path.

Tensor conventions (element strides; the last dimension must be contiguous):
    A   M x K  row-major             (torch dtype gives the element type)
    B   N x K  (the K x N matrix B stored column-major)
    C,D M x N  float32 (int32 for int8 inputs); with floating inputs also
               bfloat16, float16, float8_e4m3fn or float8_e5m2 (the epilogue
               variants: D's dtype picks the output type, C has D's dtype),
               plus an optional fp32 bias of N values and ReLU
    Ac  M x K/2, idx M x ceil(K/32) int32/uint32 words
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmmac.so")

F16, BF16, I8, FP8_E4M3, BF8_E5M2, FP4_E2M1, FP6_E2M3, BF6_E3M2 = 1, 2, 3, 4, 5, 6, 7, 8
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_MISALIGNED, ERR_HIP, ERR_SCRATCH = 0, 1, 2, 3, 4, 5

OUT_ACC, OUT_BF16, OUT_F16, OUT_FP8_E4M3, OUT_BF8_E5M2 = 0, 1, 2, 3, 4
ACT_NONE, ACT_RELU = 0, 1
OUT_OF = {torch.float32: OUT_ACC, torch.int32: OUT_ACC, torch.bfloat16: OUT_BF16, torch.float16: OUT_F16,
          torch.float8_e4m3fn: OUT_FP8_E4M3, torch.float8_e5m2: OUT_BF8_E5M2}

DTYPE_OF = {torch.float16: F16, torch.bfloat16: BF16, torch.int8: I8,
            torch.float8_e4m3fn: FP8_E4M3, torch.float8_e5m2: BF8_E5M2}
TORCH_OF = {v: k for k, v in DTYPE_OF.items()}

_lib = None


class Epilogue(ctypes.Structure):
    """mmac_epilogue_t."""
    _fields_ = [("d_type", ctypes.c_int32), ("act", ctypes.c_int32), ("bias", ctypes.c_void_p)]


class MmacError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {string(status)}")


def lib():
    """The loaded libmmac.so (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m sparse_matrix_multiply_amd.build` first")
        L = ctypes.CDLL(LIB_PATH)
        i64, dbl, vp, i32 = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
        L.mmac_gemm_dense.restype = i32
        L.mmac_gemm_dense.argtypes = [i32, i32, i64, i64, i64, dbl, vp, i64, vp, i64, dbl, vp, i64, vp, i64, vp]
        L.mmac_sparse24_compress.restype = i32
        L.mmac_sparse24_compress.argtypes = [i32, i64, i64, vp, i64, vp, i64, vp, i64, vp, vp]
        L.mmac_sparse24_prune_compress.restype = i32
        L.mmac_sparse24_prune_compress.argtypes = [i32, i64, i64, vp, i64, vp, i64, vp, i64, vp, vp]
        L.mmac_gemm_sparse24.restype = i32
        L.mmac_gemm_sparse24.argtypes = [i32, i32, i64, i64, i64, dbl, vp, i64, vp, i64, vp, i64, dbl, vp, i64,
                                         vp, i64, vp]
        ep = ctypes.POINTER(Epilogue)
        L.mmac_gemm_dense_ep.restype = i32
        L.mmac_gemm_dense_ep.argtypes = [i32, i32, i64, i64, i64, dbl, vp, i64, vp, i64, dbl, vp, i64, vp, i64, ep, vp]
        L.mmac_gemm_sparse24_ep.restype = i32
        L.mmac_gemm_sparse24_ep.argtypes = [i32, i32, i64, i64, i64, dbl, vp, i64, vp, i64, vp, i64, dbl, vp, i64,
                                            vp, i64, ep, vp]
        L.mmac_gemm_dense_ws.restype = i32
        L.mmac_gemm_dense_ws.argtypes = [i32, i32, i64, i64, i64, dbl, vp, i64, vp, i64, dbl, vp, i64, vp, i64, ep,
                                         vp, i64, vp]
        L.mmac_gemm_dense_static.restype = i32
        L.mmac_gemm_dense_static.argtypes = [i32, i32, i64, i64, i64, dbl, vp, i64, vp, i64, dbl, vp, i64, vp, i64,
                                             ep, vp]
        L.mmac_gemm_sparse24_ws.restype = i32
        L.mmac_gemm_sparse24_ws.argtypes = [i32, i32, i64, i64, i64, dbl, vp, i64, vp, i64, vp, i64, dbl, vp, i64,
                                            vp, i64, ep, vp, i64, vp]
        L.mmac_gemm_dense_mx.restype = i32
        L.mmac_gemm_dense_mx.argtypes = [i32, i32, i64, i64, i64, dbl, vp, i64, vp, i64, vp, i64, vp, i64, dbl, vp,
                                         i64, vp, i64, ep, vp]
        L.mmac_gemm_dense_layout.restype = i32
        L.mmac_gemm_dense_layout.argtypes = [i32, i32, i32, i32, i64, i64, i64, dbl, vp, i64, vp, i64, dbl, vp, i64,
                                             vp, i64, ep, vp]
        L.mmac_gemm_workspace_bytes.restype = i64
        L.mmac_gemm_workspace_bytes.argtypes = [i32, i64, i64, i64, i32]
        L.mmac_status_string.restype = ctypes.c_char_p
        L.mmac_status_string.argtypes = [i32]
        _lib = L
    return _lib


def string(status):
    return lib().mmac_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ld(t):
    """Row pitch (elements) of a 2-D tensor whose last dimension is contiguous and whose rows do not
    overlap (a broadcast or overlapping view would make the kernels write past or over its rows)."""
    st, sh = t.stride(), t.shape
    if len(sh) != 2 or (st[1] != 1 and sh[1] > 1):
        raise ValueError("expected a 2-D tensor with a contiguous last dimension")
    if sh[0] > 1 and st[0] < sh[1]:
        raise ValueError(f"rows of a {tuple(sh)} tensor with row stride {st[0]} overlap")
    return max(st[0], sh[1], 1)


def _shape(t, rows, cols, name, min_cols=False):
    """Check that a 2-D tensor has `rows` rows and `cols` columns (at least `cols` with min_cols)."""
    if t is None:
        return
    if t.dim() != 2 or t.shape[0] != rows or (t.shape[1] < cols if min_cols else t.shape[1] != cols):
        want = f"({rows}, {'>= ' if min_cols else ''}{cols})"
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {want}")


def _same_device(*tensors):
    """Every tensor given lives on one CUDA device (the library's kernels address them all)."""
    devs = {t.device for t in tensors if t is not None}
    if any(d.type != "cuda" for d in devs):
        raise ValueError("every tensor must be in GPU memory")
    if len(devs) > 1:
        raise ValueError(f"tensors on different devices: {sorted(str(d) for d in devs)}")


def _bias(bias, N):
    if bias is not None and (bias.dtype != torch.float32 or bias.dim() != 1 or bias.numel() < N or
                             (bias.numel() > 1 and bias.stride(0) != 1)):
        raise ValueError(f"bias must be a contiguous float32 vector of at least N = {N} values")


# The current stream's handle without building a Stream object (a few microseconds per call, which
# is as long as a small GEMM): torch's own accessor where it has one.
_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream):
    if stream is None:
        if _raw_current_stream is not None:
            return ctypes.c_void_p(_raw_current_stream(torch.cuda.current_device()))
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype(t, given):
    return given if given is not None else DTYPE_OF[t.dtype]


def _check(status, what):
    if status != OK:
        raise MmacError(status, what)


def _epilogue(D, bias, act, d_type, C=None):
    """The mmac_epilogue_t of a call, or None for the plain call.  D (and C) must have the element
    size of the output type the call writes."""
    if d_type is None:
        if D.dtype not in OUT_OF:
            raise ValueError(f"D has dtype {D.dtype}; expected one of {sorted(str(t) for t in OUT_OF)}")
        d_type = OUT_OF[D.dtype]
    size = {OUT_ACC: 4, OUT_BF16: 2, OUT_F16: 2, OUT_FP8_E4M3: 1, OUT_BF8_E5M2: 1}.get(d_type)
    for t, name in ((D, "D"), (C, "C")):
        if size is not None and t is not None and t.element_size() != size:
            raise ValueError(f"{name} has {t.element_size()}-byte elements; the output type writes {size}")
    if d_type == OUT_ACC and bias is None and act == ACT_NONE:
        return None
    return Epilogue(d_type, act, None if bias is None else bias.data_ptr())


def workspace_bytes(a_type, M, N, K, sparse=False):
    """Bytes of workspace the split-K calls use for this product (0: they would not split)."""
    return int(lib().mmac_gemm_workspace_bytes(int(a_type), M, N, K, 1 if sparse else 0))


def workspace(a_type, M, N, K, sparse=False, device=None):
    """A zeroed workspace tensor for the split-K calls (None if they would not split)."""
    n = workspace_bytes(a_type, M, N, K, sparse)
    if n == 0:
        return None
    return torch.zeros(n, dtype=torch.uint8, device=device if device is not None else torch.device("cuda"))


def gemm_dense(A, B, D, alpha=1.0, beta=0.0, C=None, a_type=None, b_type=None, stream=None, bias=None,
               act=ACT_NONE, d_type=None, workspace=None):
    """D = alpha * A @ B + beta * C with A M x K (row-major) and B given as its N x K transpose.
    With bias (N fp32 values), act or a bfloat16 / float16 D (d_type overrides what D's dtype
    says) this is mmac_gemm_dense_ep: D = round(act(alpha * A @ B + beta * C + bias)); with a
    workspace tensor (see workspace()) it is mmac_gemm_dense_ws, which may split K."""
    M, K = A.shape
    N = B.shape[0]
    _shape(B, N, K, "B")
    _shape(D, M, N, "D")
    _shape(C, M, N, "C")
    _bias(bias, N)
    _same_device(A, B, C, D, bias, workspace)
    ta, tb = _dtype(A, a_type), _dtype(B, b_type)
    args = (ta, tb, M, N, K, float(alpha), _ptr(A), _ld(A), _ptr(B), _ld(B), float(beta),
            _ptr(C), _ld(C) if C is not None else 0, _ptr(D), _ld(D))
    ep = _epilogue(D, bias, act, d_type, C)
    if workspace is not None:
        _check(lib().mmac_gemm_dense_ws(*args, None if ep is None else ctypes.byref(ep), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream)),
               "mmac_gemm_dense_ws")
    elif ep is None:
        _check(lib().mmac_gemm_dense(*args, _stream(stream)), "mmac_gemm_dense")
    else:
        _check(lib().mmac_gemm_dense_ep(*args, ctypes.byref(ep), _stream(stream)), "mmac_gemm_dense_ep")
    return D


def _compress_shapes(A, Ac, idx, bad_groups):
    M, K = A.shape
    _shape(Ac, M, K // 2, "Ac")
    _shape(idx, M, (K + 31) // 32, "idx")
    if idx.element_size() != 4:
        raise ValueError("idx must hold 32-bit words")
    if bad_groups is not None and (bad_groups.numel() < 1 or bad_groups.element_size() != 4):
        raise ValueError("bad_groups must hold at least one 32-bit counter")
    _same_device(A, Ac, idx, bad_groups)


def gemm_dense_static(A, B, D, alpha=1.0, beta=0.0, C=None, a_type=None, b_type=None, stream=None, bias=None,
                      act=ACT_NONE, d_type=None):
    """gemm_dense with split-K through the library's fixed scratch array (mmac_gemm_dense_static):
    no workspace argument, nothing allocated."""
    M, K = A.shape
    N = B.shape[0]
    _shape(B, N, K, "B")
    _shape(D, M, N, "D")
    _shape(C, M, N, "C")
    _bias(bias, N)
    _same_device(A, B, C, D, bias)
    ta, tb = _dtype(A, a_type), _dtype(B, b_type)
    ep = _epilogue(D, bias, act, d_type, C)
    _check(lib().mmac_gemm_dense_static(ta, tb, M, N, K, float(alpha), _ptr(A), _ld(A), _ptr(B), _ld(B), float(beta),
                                        _ptr(C), _ld(C) if C is not None else 0, _ptr(D), _ld(D),
                                        None if ep is None else ctypes.byref(ep), _stream(stream)),
           "mmac_gemm_dense_static")
    return D


def sparse24_compress(A, Ac, idx, bad_groups=None, a_type=None, stream=None):
    """Compress a 4:2 A (M x K) into Ac (M x K/2) and idx (M x ceil(K/32) words)."""
    M, K = A.shape
    _compress_shapes(A, Ac, idx, bad_groups)
    ta = _dtype(A, a_type)
    st = lib().mmac_sparse24_compress(ta, M, K, _ptr(A), _ld(A), _ptr(Ac), _ld(Ac), _ptr(idx), _ld(idx),
                                      _ptr(bad_groups), _stream(stream))
    _check(st, "mmac_sparse24_compress")
    return Ac, idx


def sparse24_prune_compress(A, Ac, idx, bad_groups=None, a_type=None, stream=None):
    """Prune a dense A (M x K) to 4:2 by magnitude (two largest |a| per group of four) and
    compress it into Ac (M x K/2) and idx (M x ceil(K/32) words), in one pass."""
    M, K = A.shape
    _compress_shapes(A, Ac, idx, bad_groups)
    ta = _dtype(A, a_type)
    st = lib().mmac_sparse24_prune_compress(ta, M, K, _ptr(A), _ld(A), _ptr(Ac), _ld(Ac), _ptr(idx), _ld(idx),
                                            _ptr(bad_groups), _stream(stream))
    _check(st, "mmac_sparse24_prune_compress")
    return Ac, idx


def gemm_sparse24(Ac, idx, B, D, K=None, alpha=1.0, beta=0.0, C=None, a_type=None, b_type=None, stream=None,
                  bias=None, act=ACT_NONE, d_type=None, workspace=None):
    """D = alpha * A @ B + beta * C with A given compressed (Ac, idx); K is the dense K.
    bias / act / a 16-bit D select mmac_gemm_sparse24_ep and a workspace mmac_gemm_sparse24_ws,
    as in gemm_dense."""
    M = Ac.shape[0]
    N, KB = B.shape
    K = KB if K is None else K
    _shape(Ac, M, K // 2, "Ac")
    _shape(B, N, K, "B")
    _shape(idx, M, (K + 31) // 32, "idx", min_cols=True)
    if idx.element_size() != 4:
        raise ValueError("idx must hold 32-bit words")
    _shape(D, M, N, "D")
    _shape(C, M, N, "C")
    _bias(bias, N)
    _same_device(Ac, idx, B, C, D, bias, workspace)
    ta, tb = _dtype(Ac, a_type), _dtype(B, b_type)
    args = (ta, tb, M, N, K, float(alpha), _ptr(Ac), _ld(Ac), _ptr(idx), _ld(idx), _ptr(B), _ld(B), float(beta),
            _ptr(C), _ld(C) if C is not None else 0, _ptr(D), _ld(D))
    ep = _epilogue(D, bias, act, d_type, C)
    if workspace is not None:
        _check(lib().mmac_gemm_sparse24_ws(*args, None if ep is None else ctypes.byref(ep), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _stream(stream)),
               "mmac_gemm_sparse24_ws")
    elif ep is None:
        _check(lib().mmac_gemm_sparse24(*args, _stream(stream)), "mmac_gemm_sparse24")
    else:
        _check(lib().mmac_gemm_sparse24_ep(*args, ctypes.byref(ep), _stream(stream)), "mmac_gemm_sparse24_ep")
    return D


def gemm_mx(A, SA, B, SB, D, alpha=1.0, beta=0.0, C=None, a_type=None, b_type=None, stream=None, bias=None,
            act=ACT_NONE, d_type=None):
    """Block-scaled (MX) GEMM: D = alpha * (A, SA) @ (B, SB) + beta * C.  A M x K and B N x K fp8;
    SA and SB the E8M0 scale words (ceil(K/128) x >= M and ceil(K/128) x >= N int32 tensors,
    four block exponents per word, see include/mmac.h).  For FP4_E2M1, A and B are uint8 tensors
    of packed pairs (M x K/2, N x K/2); for FP6_E2M3 / BF6_E3M2 uint8 tensors of packed
    elements, four per three bytes (M x 3K/4, N x 3K/4).  Epilogue arguments as in gemm_dense."""
    M, K = A.shape
    N = B.shape[0]
    ta, tb = _dtype(A, a_type), _dtype(B, b_type)

    def elems(nbytes, t):                      # elements in nbytes stored bytes of type t
        if t == FP4_E2M1:
            return nbytes * 2
        if t in (FP6_E2M3, BF6_E3M2):
            if nbytes % 3:
                raise ValueError("packed FP6 rows and pitches must be whole multiples of 3 bytes")
            return nbytes // 3 * 4
        return nbytes

    K, lda, ldb = elems(K, ta), elems(_ld(A), ta), elems(_ld(B), tb)
    if elems(B.shape[1], tb) != K:
        raise ValueError(f"B has {elems(B.shape[1], tb)} elements per row, A has {K}")
    _shape(SA, (K + 127) // 128, M, "SA", min_cols=True)
    _shape(SB, (K + 127) // 128, N, "SB", min_cols=True)
    if SA.element_size() != 4 or SB.element_size() != 4:
        raise ValueError("SA and SB must hold 32-bit scale words")
    _shape(D, M, N, "D")
    _shape(C, M, N, "C")
    _bias(bias, N)
    _same_device(A, SA, B, SB, C, D, bias)
    ep = _epilogue(D, bias, act, d_type, C)
    st = lib().mmac_gemm_dense_mx(ta, tb, M, N, K, float(alpha), _ptr(A), lda, _ptr(SA), _ld(SA), _ptr(B), ldb,
                                  _ptr(SB), _ld(SB), float(beta), _ptr(C), _ld(C) if C is not None else 0, _ptr(D),
                                  _ld(D), None if ep is None else ctypes.byref(ep), _stream(stream))
    _check(st, "mmac_gemm_dense_mx")
    return D


def gemm_layout(A, B, D, trans_a=False, trans_b=False, alpha=1.0, beta=0.0, C=None, a_type=None, b_type=None,
                stream=None, bias=None, act=ACT_NONE, d_type=None):
    """D = alpha * op(A) @ op(B) + beta * C for every dense type pair.  trans_a: A is given as its K x M
    transpose (M contiguous); trans_b: B is given as K x N (N contiguous).  Otherwise A is M x K and
    B is N x K as in gemm_dense."""
    M = A.shape[1] if trans_a else A.shape[0]
    K = A.shape[0] if trans_a else A.shape[1]
    N = B.shape[1] if trans_b else B.shape[0]
    if (B.shape[0] if trans_b else B.shape[1]) != K:
        raise ValueError(f"B has shape {tuple(B.shape)}, which does not hold K = {K} for this layout")
    _shape(D, M, N, "D")
    _shape(C, M, N, "C")
    _bias(bias, N)
    _same_device(A, B, C, D, bias)
    ta, tb = _dtype(A, a_type), _dtype(B, b_type)
    ep = _epilogue(D, bias, act, d_type, C)
    st = lib().mmac_gemm_dense_layout(ta, tb, int(bool(trans_a)), int(bool(trans_b)), M, N, K, float(alpha), _ptr(A),
                                      _ld(A), _ptr(B), _ld(B), float(beta), _ptr(C), _ld(C) if C is not None else 0,
                                      _ptr(D), _ld(D), None if ep is None else ctypes.byref(ep), _stream(stream))
    _check(st, "mmac_gemm_dense_layout")
    return D


def raw_call(name, *args):
    """Call a C entry point with raw arguments (pointers as ints); returns the status."""
    return getattr(lib(), name)(*args)
