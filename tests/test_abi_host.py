"""Host-side checks of the C ABI (no GPU needed, no compute call).

- libmmac.so loads and exports every function include/mmac.h declares;
- the status strings exist;
- every argument error is reported before any GPU work (the pointers passed
  here are fake, so these calls must return before touching the device).
"""
import ctypes
import os
import re

import pytest

import sparse_matrix_multiply_amd as mm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mmac.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mmac_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mm.LIB_PATH):
        from sparse_matrix_multiply_amd import build
        build.build()
    return mm.lib()


def test_header_declares_the_entry_points():
    assert declared_functions() == ["mmac_gemm_dense", "mmac_gemm_dense_ep", "mmac_gemm_dense_layout",
                                    "mmac_gemm_dense_mx", "mmac_gemm_dense_static",
                                    "mmac_gemm_dense_ws",
                                    "mmac_gemm_sparse24", "mmac_gemm_sparse24_ep", "mmac_gemm_sparse24_ws",
                                    "mmac_gemm_workspace_bytes", "mmac_sparse24_compress",
                                    "mmac_sparse24_prune_compress", "mmac_status_string"]


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings(L):
    for s in range(6):
        assert mm.string(s).startswith(["MMAC_OK", "MMAC_ERR_INVALID_ARG", "MMAC_ERR_UNSUPPORTED",
                                        "MMAC_ERR_MISALIGNED", "MMAC_ERR_HIP", "MMAC_ERR_SCRATCH"][s])
    assert mm.string(99) == "unknown mmac status"


P = 1 << 20          # a fake, 16-byte aligned "device pointer": never dereferenced here


def dense(L, **kw):
    a = dict(a=mm.BF16, b=mm.BF16, M=64, N=64, K=64, alpha=1.0, A=P, lda=64, B=P, ldb=64, beta=0.0,
             C=None, ldc=64, D=P, ldd=64, stream=None)
    a.update(kw)
    return L.mmac_gemm_dense(a["a"], a["b"], a["M"], a["N"], a["K"], a["alpha"], a["A"], a["lda"], a["B"],
                             a["ldb"], a["beta"], a["C"], a["ldc"], a["D"], a["ldd"], a["stream"])


def sparse(L, **kw):
    a = dict(a=mm.F16, b=mm.F16, M=64, N=64, K=64, alpha=1.0, Ac=P, ldac=32, idx=P, ldidx=2, B=P, ldb=64,
             beta=0.0, C=None, ldc=64, D=P, ldd=64, stream=None)
    a.update(kw)
    return L.mmac_gemm_sparse24(a["a"], a["b"], a["M"], a["N"], a["K"], a["alpha"], a["Ac"], a["ldac"],
                                a["idx"], a["ldidx"], a["B"], a["ldb"], a["beta"], a["C"], a["ldc"], a["D"],
                                a["ldd"], a["stream"])


def compress(L, entry="mmac_sparse24_compress", **kw):
    a = dict(a=mm.F16, M=64, K=64, A=P, lda=64, Ac=P, ldac=32, idx=P, ldidx=2, bad=None, stream=None)
    a.update(kw)
    return getattr(L, entry)(a["a"], a["M"], a["K"], a["A"], a["lda"], a["Ac"], a["ldac"], a["idx"],
                             a["ldidx"], a["bad"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(a=mm.BF16, b=mm.F16), mm.ERR_UNSUPPORTED),
    (dict(a=mm.I8, b=mm.BF16), mm.ERR_UNSUPPORTED),
    (dict(a=mm.FP8_E4M3, b=mm.I8), mm.ERR_UNSUPPORTED),
    (dict(a=0, b=0), mm.ERR_UNSUPPORTED),
    (dict(a=6, b=6), mm.ERR_UNSUPPORTED),
    (dict(M=-1), mm.ERR_INVALID_ARG),
    (dict(K=-5), mm.ERR_INVALID_ARG),
    (dict(N=1 << 31), mm.ERR_INVALID_ARG),
    (dict(A=None), mm.ERR_INVALID_ARG),
    (dict(B=None), mm.ERR_INVALID_ARG),
    (dict(D=None), mm.ERR_INVALID_ARG),
    (dict(beta=1.0, C=None), mm.ERR_INVALID_ARG),
    (dict(lda=32), mm.ERR_INVALID_ARG),
    (dict(ldb=8), mm.ERR_INVALID_ARG),
    (dict(ldd=63), mm.ERR_INVALID_ARG),
    (dict(beta=1.0, C=P + 4096, ldc=32), mm.ERR_INVALID_ARG),
    (dict(beta=1.0, C=P, ldc=64, ldd=128), mm.ERR_INVALID_ARG),        # in place needs ldc == ldd
    (dict(alpha=float("nan")), mm.ERR_INVALID_ARG),
    (dict(alpha=float("inf")), mm.ERR_INVALID_ARG),
    (dict(alpha=3.5e38), mm.ERR_INVALID_ARG),                           # finite double, beyond fp32
    (dict(beta=-1e300, C=P + 4096), mm.ERR_INVALID_ARG),
    (dict(a=mm.I8, b=mm.I8, alpha=1.5), mm.ERR_INVALID_ARG),
    (dict(a=mm.I8, b=mm.I8, beta=2.0 ** 31, C=P + 4096), mm.ERR_INVALID_ARG),
    (dict(A=P + 8), mm.ERR_MISALIGNED),
    (dict(B=P + 2), mm.ERR_MISALIGNED),
    (dict(lda=68), mm.ERR_MISALIGNED),                                 # 136-byte pitch
    (dict(D=P + 2), mm.ERR_MISALIGNED),
    (dict(lda=(1 << 23)), mm.ERR_UNSUPPORTED),                         # 16 MiB row pitch
])
def test_dense_argument_errors(L, kw, code):
    assert dense(L, **kw) == code


def test_dense_empty_is_a_no_op(L):
    assert dense(L, M=0) == mm.OK
    assert dense(L, N=0) == mm.OK


@pytest.mark.parametrize("kw,code", [
    (dict(K=66), mm.ERR_INVALID_ARG),                                  # K % 4 != 0
    (dict(ldac=16), mm.ERR_INVALID_ARG),
    (dict(idx=None), mm.ERR_INVALID_ARG),
    (dict(ldidx=1), mm.ERR_INVALID_ARG),
    (dict(a=mm.F16, b=mm.BF16), mm.ERR_UNSUPPORTED),
    (dict(Ac=P + 4), mm.ERR_MISALIGNED),
    (dict(idx=P + 2), mm.ERR_MISALIGNED),
])
def test_sparse_argument_errors(L, kw, code):
    assert sparse(L, **kw) == code


def test_sparse_empty_is_a_no_op(L):
    assert sparse(L, M=0) == mm.OK


@pytest.mark.parametrize("kw,code", [
    (dict(K=30), mm.ERR_INVALID_ARG),
    (dict(a=9), mm.ERR_UNSUPPORTED),
    (dict(A=None), mm.ERR_INVALID_ARG),
    (dict(lda=60), mm.ERR_INVALID_ARG),
    (dict(ldidx=1), mm.ERR_INVALID_ARG),
    (dict(A=P + 8), mm.ERR_MISALIGNED),
    (dict(ldac=36), mm.ERR_MISALIGNED),
    (dict(bad=P + 1), mm.ERR_MISALIGNED),
])
@pytest.mark.parametrize("entry", ["mmac_sparse24_compress", "mmac_sparse24_prune_compress"])
def test_compress_argument_errors(L, kw, code, entry):
    assert compress(L, entry, **kw) == code


@pytest.mark.parametrize("entry", ["mmac_sparse24_compress", "mmac_sparse24_prune_compress"])
def test_compress_empty_is_a_no_op(L, entry):
    assert compress(L, entry, M=0) == mm.OK
    assert compress(L, entry, K=0, ldidx=1, lda=8, ldac=8) == mm.OK


def dense_ep(L, ep, **kw):
    a = dict(a=mm.BF16, b=mm.BF16, M=64, N=64, K=64, alpha=1.0, A=P, lda=64, B=P, ldb=64, beta=0.0,
             C=None, ldc=64, D=P, ldd=64, stream=None)
    a.update(kw)
    return L.mmac_gemm_dense_ep(a["a"], a["b"], a["M"], a["N"], a["K"], a["alpha"], a["A"], a["lda"], a["B"],
                                a["ldb"], a["beta"], a["C"], a["ldc"], a["D"], a["ldd"],
                                None if ep is None else ctypes.byref(ep), a["stream"])


def sparse_ep(L, ep, **kw):
    a = dict(a=mm.F16, b=mm.F16, M=64, N=64, K=64, alpha=1.0, Ac=P, ldac=32, idx=P, ldidx=2, B=P, ldb=64,
             beta=0.0, C=None, ldc=64, D=P, ldd=64, stream=None)
    a.update(kw)
    return L.mmac_gemm_sparse24_ep(a["a"], a["b"], a["M"], a["N"], a["K"], a["alpha"], a["Ac"], a["ldac"],
                                   a["idx"], a["ldidx"], a["B"], a["ldb"], a["beta"], a["C"], a["ldc"], a["D"],
                                   a["ldd"], None if ep is None else ctypes.byref(ep), a["stream"])


EP_ERRORS = [
    (dict(d_type=5), {}, mm.ERR_INVALID_ARG),
    (dict(d_type=-1), {}, mm.ERR_INVALID_ARG),
    (dict(act=2), {}, mm.ERR_INVALID_ARG),
    (dict(bias=P + 2), {}, mm.ERR_MISALIGNED),
    (dict(d_type=mm.OUT_BF16), dict(D=P + 1), mm.ERR_MISALIGNED),                 # 2-byte D, odd address
    (dict(d_type=mm.OUT_F16), dict(beta=1.0, C=P + 4097), mm.ERR_MISALIGNED),
    (dict(d_type=mm.OUT_F16), dict(ldd=(1 << 22) + 1, N=64), mm.ERR_UNSUPPORTED),  # > 8 MiB of binary16
    (dict(d_type=mm.OUT_BF8_E5M2), dict(ldd=(1 << 23) + 1, N=64), mm.ERR_UNSUPPORTED),  # > 8 MiB of bytes
    (dict(d_type=mm.OUT_FP8_E4M3), dict(a=mm.I8, b=mm.I8), mm.ERR_UNSUPPORTED),
    (dict(d_type=mm.OUT_BF16), dict(a=mm.I8, b=mm.I8), mm.ERR_UNSUPPORTED),       # int8: plain output only
    (dict(act=mm.ACT_RELU), dict(a=mm.I8, b=mm.I8), mm.ERR_UNSUPPORTED),
    (dict(bias=P), dict(a=mm.I8, b=mm.I8), mm.ERR_UNSUPPORTED),
    (dict(), dict(ldd=63), mm.ERR_INVALID_ARG),                                   # plain checks still apply
]


@pytest.mark.parametrize("epkw,kw,code", EP_ERRORS)
def test_epilogue_argument_errors(L, epkw, kw, code):
    ep = mm.Epilogue(epkw.get("d_type", mm.OUT_ACC), epkw.get("act", mm.ACT_NONE), epkw.get("bias"))
    assert dense_ep(L, ep, **kw) == code
    if kw.get("a") != mm.I8:
        assert sparse_ep(L, ep, **kw) == code


def test_epilogue_null_and_empty(L):
    # NULL epilogue = the plain call (same checks); empty outputs are a no-op for every variant
    assert dense_ep(L, None, ldd=63) == mm.ERR_INVALID_ARG
    assert sparse_ep(L, None, K=66) == mm.ERR_INVALID_ARG
    for d in (mm.OUT_ACC, mm.OUT_BF16, mm.OUT_F16, mm.OUT_FP8_E4M3, mm.OUT_BF8_E5M2):
        ep = mm.Epilogue(d, mm.ACT_RELU, P)
        assert dense_ep(L, ep, M=0) == mm.OK
        assert sparse_ep(L, ep, N=0) == mm.OK


def dense_ws(L, ws, ws_bytes, **kw):
    a = dict(a=mm.BF16, b=mm.BF16, M=8192, N=1024, K=8192, alpha=1.0, A=P, lda=8192, B=P, ldb=8192, beta=0.0,
             C=None, ldc=1024, D=P, ldd=1024, stream=None)
    a.update(kw)
    return L.mmac_gemm_dense_ws(a["a"], a["b"], a["M"], a["N"], a["K"], a["alpha"], a["A"], a["lda"], a["B"],
                                a["ldb"], a["beta"], a["C"], a["ldc"], a["D"], a["ldd"], None, ws, ws_bytes,
                                a["stream"])


def test_workspace_bytes_plan(L, monkeypatch):
    monkeypatch.delenv("MMAC_SPLITK", raising=False)
    monkeypatch.delenv("MMAC_TILE", raising=False)
    T64 = 64 * 64 * 4                                    # bytes of one fp32 64 x 64 partial tile
    # 512 x 512 in 64 x 64 tiles: 64 tiles, so four K ranges (counters padded to 256 bytes)
    assert mm.workspace_bytes(mm.BF16, 512, 512, 32768) == 256 + 4 * 64 * T64
    # 256 x 256: 16 tiles, at most eight ranges; 1024 x 512: 128 tiles (512 counter bytes), two ranges
    assert mm.workspace_bytes(mm.BF16, 256, 256, 65536) == 256 + 8 * 16 * T64
    assert mm.workspace_bytes(mm.FP8_E4M3, 1024, 512, 8192) == 512 + 2 * 128 * T64
    assert mm.workspace_bytes(mm.FP8_E4M3, 1024, 512, 8192, sparse=True) == 512 + 2 * 128 * T64
    # about one tile per compute unit already, the skinny path, too little K, empty: no split
    assert mm.workspace_bytes(mm.BF16, 8192, 1024, 8192) == 0
    assert mm.workspace_bytes(mm.BF16, 8192, 8192, 8192) == 0
    assert mm.workspace_bytes(mm.BF16, 16, 4096, 4096) == 0
    assert mm.workspace_bytes(mm.BF16, 512, 512, 256) == 0
    assert mm.workspace_bytes(mm.BF16, 0, 1024, 8192) == 0
    # forced: three ranges of the 256 x 256 tiles of an 8192^3 product
    monkeypatch.setenv("MMAC_SPLITK", "3")
    assert mm.workspace_bytes(mm.BF16, 8192, 8192, 8192) == 4096 + 3 * 1024 * 256 * 256 * 4


@pytest.mark.parametrize("ws,nbytes,code", [
    (P + 8, 1 << 30, mm.ERR_MISALIGNED),
    (P, -1, mm.ERR_INVALID_ARG),
])
def test_workspace_argument_errors(L, ws, nbytes, code):
    assert dense_ws(L, ws, nbytes) == code
    assert dense_ws(L, ws, nbytes, M=0) == code        # checked before the empty-output shortcut


def test_workspace_calls_validate_like_the_plain_ones(L):
    assert dense_ws(L, None, 0, ldd=1000) == mm.ERR_INVALID_ARG
    assert dense_ws(L, None, 0, M=0) == mm.OK


def dense_mx(L, **kw):
    a = dict(a=mm.FP8_E4M3, b=mm.BF8_E5M2, M=64, N=64, K=256, alpha=1.0, A=P, lda=256, SA=P, ldsa=64, B=P, ldb=256,
             SB=P, ldsb=64, beta=0.0, C=None, ldc=64, D=P, ldd=64, stream=None)
    a.update(kw)
    return L.mmac_gemm_dense_mx(a["a"], a["b"], a["M"], a["N"], a["K"], a["alpha"], a["A"], a["lda"], a["SA"],
                                a["ldsa"], a["B"], a["ldb"], a["SB"], a["ldsb"], a["beta"], a["C"], a["ldc"], a["D"],
                                a["ldd"], None, a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(a=mm.BF16, b=mm.BF16), mm.ERR_UNSUPPORTED),
    (dict(a=mm.I8, b=mm.I8), mm.ERR_UNSUPPORTED),
    (dict(a=mm.FP8_E4M3, b=mm.BF16), mm.ERR_UNSUPPORTED),
    (dict(K=48, lda=64, ldb=64), mm.ERR_INVALID_ARG),                 # K % 32 != 0
    (dict(SA=None), mm.ERR_INVALID_ARG),
    (dict(SB=None), mm.ERR_INVALID_ARG),
    (dict(ldsa=60), mm.ERR_INVALID_ARG),                             # < M
    (dict(ldsb=62, N=60, ldd=64), mm.ERR_MISALIGNED),                 # ldsb % 4
    (dict(SA=P + 4), mm.ERR_MISALIGNED),
    (dict(SB=P + 8), mm.ERR_MISALIGNED),
    (dict(lda=200), mm.ERR_INVALID_ARG),
    (dict(a=mm.FP4_E2M1, b=mm.FP8_E4M3), mm.ERR_UNSUPPORTED),         # FP4 only with FP4
    (dict(a=mm.FP4_E2M1, b=mm.FP4_E2M1, lda=257, ldb=256), mm.ERR_MISALIGNED),   # odd element pitch
    (dict(a=mm.FP4_E2M1, b=mm.FP4_E2M1, lda=264, ldb=256), mm.ERR_MISALIGNED),   # 132-byte rows
    (dict(a=mm.FP4_E2M1, b=mm.FP4_E2M1, lda=128, ldb=256), mm.ERR_INVALID_ARG),  # lda < K
    (dict(a=mm.FP6_E2M3, b=mm.FP8_E4M3), mm.ERR_UNSUPPORTED),         # FP6 only with FP6
    (dict(a=mm.FP8_E4M3, b=mm.BF6_E3M2), mm.ERR_UNSUPPORTED),
    (dict(a=mm.FP6_E2M3, b=mm.FP4_E2M1), mm.ERR_UNSUPPORTED),
    (dict(a=mm.FP6_E2M3, b=mm.BF6_E3M2, lda=258), mm.ERR_MISALIGNED),   # not whole bytes
    (dict(a=mm.BF6_E3M2, b=mm.FP6_E2M3, ldb=260), mm.ERR_MISALIGNED),   # 195-byte rows
    (dict(a=mm.FP6_E2M3, b=mm.FP6_E2M3, lda=192), mm.ERR_INVALID_ARG),  # lda < K (144-byte rows)
    (dict(a=mm.FP6_E2M3, b=mm.FP6_E2M3, K=240, lda=256, ldb=256), mm.ERR_INVALID_ARG),   # K % 32
])
def test_mx_argument_errors(L, kw, code):
    assert dense_mx(L, **kw) == code


def test_mx_empty_is_a_no_op(L):
    assert dense_mx(L, M=0) == mm.OK
    assert dense_mx(L, N=0) == mm.OK
    assert dense_mx(L, M=0, a=mm.FP4_E2M1, b=mm.FP4_E2M1) == mm.OK
    assert dense_mx(L, M=0, a=mm.FP6_E2M3, b=mm.BF6_E3M2) == mm.OK


def test_fp4_and_fp6_are_only_for_block_scaled_gemm(L):
    assert dense(L, a=mm.FP4_E2M1, b=mm.FP4_E2M1) == mm.ERR_UNSUPPORTED
    assert compress(L, a=mm.FP4_E2M1) == mm.ERR_UNSUPPORTED
    for t in (mm.FP6_E2M3, mm.BF6_E3M2):
        assert dense(L, a=t, b=t) == mm.ERR_UNSUPPORTED
        assert compress(L, a=t) == mm.ERR_UNSUPPORTED


def dense_layout(L, **kw):
    a = dict(a=mm.BF16, b=mm.BF16, ta=1, tb=0, M=64, N=64, K=64, alpha=1.0, A=P, lda=64, B=P, ldb=64, beta=0.0,
             C=None, ldc=64, D=P, ldd=64, stream=None)
    a.update(kw)
    return L.mmac_gemm_dense_layout(a["a"], a["b"], a["ta"], a["tb"], a["M"], a["N"], a["K"], a["alpha"], a["A"],
                                    a["lda"], a["B"], a["ldb"], a["beta"], a["C"], a["ldc"], a["D"], a["ldd"], None,
                                    a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(ta=2), mm.ERR_INVALID_ARG),
    (dict(tb=-1), mm.ERR_INVALID_ARG),
    (dict(a=mm.FP8_E4M3, b=mm.BF16), mm.ERR_UNSUPPORTED),
    (dict(a=mm.I8, b=mm.FP8_E4M3, ta=0, tb=1), mm.ERR_UNSUPPORTED),
    (dict(a=mm.FP4_E2M1, b=mm.FP4_E2M1), mm.ERR_UNSUPPORTED),         # block-scaled formats: MX entry only
    (dict(a=mm.I8, b=mm.I8, alpha=1.5), mm.ERR_INVALID_ARG),          # int8: integer alpha
    (dict(a=mm.I8, b=mm.I8, M=48, lda=56, ldd=64), mm.ERR_MISALIGNED),   # 56-byte rows of int8
    (dict(a=mm.FP8_E4M3, b=mm.BF8_E5M2, K=1 << 21, lda=1 << 10, ldb=1 << 21), mm.ERR_UNSUPPORTED),  # 2 GiB of A
    (dict(M=100, lda=96), mm.ERR_INVALID_ARG),                        # trans A: lda >= M
    (dict(ta=0, tb=1, N=100, ldb=96, ldd=100), mm.ERR_INVALID_ARG),     # trans B: ldb >= N
    (dict(M=60, lda=60, ldd=64), mm.ERR_MISALIGNED),                  # 120-byte rows
    (dict(K=1 << 20, lda=1 << 12, ldb=1 << 20), mm.ERR_UNSUPPORTED),   # 8 GiB of transposed A
    (dict(ta=0, lda=32), mm.ERR_INVALID_ARG),                         # plain checks when not transposed
])
def test_layout_argument_errors(L, kw, code):
    assert dense_layout(L, **kw) == code


def test_layout_empty_is_a_no_op(L):
    assert dense_layout(L, M=0) == mm.OK
    assert dense_layout(L, N=0, tb=1) == mm.OK


def test_binding_rejects_partial_fp6_rows():
    """The Python binding counts packed-FP6 rows and pitches in whole 3-byte groups of four
    elements; anything else is refused before the library is called."""
    import torch
    A = torch.zeros((4, 50), dtype=torch.uint8)            # 50 bytes: not a whole number of elements
    B = torch.zeros((4, 48), dtype=torch.uint8)
    S = torch.zeros((1, 4), dtype=torch.int32)
    D = torch.zeros((4, 4), dtype=torch.float32)
    with pytest.raises(ValueError):
        mm.gemm_mx(A, S, B, S, D, a_type=mm.FP6_E2M3, b_type=mm.FP6_E2M3)
    with pytest.raises(ValueError):
        mm.gemm_mx(B, S, A, S, D, a_type=mm.BF6_E3M2, b_type=mm.FP6_E2M3)


def test_binding_checks_shapes_before_any_launch():
    """The binding rejects tensors whose shapes, strides or element sizes do not match the call
    (the kernels would otherwise write outside the caller's buffers); host tensors suffice, since
    every check runs before the library is called."""
    import torch
    A = torch.zeros((64, 128), dtype=torch.bfloat16)
    B = torch.zeros((32, 128), dtype=torch.bfloat16)
    D = torch.zeros((64, 32), dtype=torch.float32)
    bad = [
        dict(D=torch.zeros((63, 32))),                                 # too few rows of D
        dict(D=torch.zeros((64, 31))),
        dict(D=torch.zeros((64, 32), dtype=torch.int16)),              # 2-byte D for a 4-byte output
        dict(D=torch.zeros((64, 32), dtype=torch.float64)),
        dict(C=torch.zeros((32, 32)), beta=1.0),
        dict(B=torch.zeros((32, 64), dtype=torch.bfloat16)),           # K mismatch
        dict(bias=torch.zeros(16)),                                    # bias shorter than N
        dict(bias=torch.zeros(32, dtype=torch.float16)),
        dict(D=torch.zeros((1, 32)).expand(64, 32)),                   # rows overlap (stride 0)
    ]
    for kw in bad:
        args = dict(A=A, B=B, D=D)
        args.update(kw)
        with pytest.raises(ValueError):
            mm.gemm_dense(**args)
    with pytest.raises(ValueError):                                    # host memory
        mm.gemm_dense(A, B, D)

    Ac = torch.zeros((64, 64), dtype=torch.float16)
    idx = torch.zeros((64, 4), dtype=torch.int32)
    Bs = torch.zeros((32, 128), dtype=torch.float16)
    for kw in (dict(Ac=torch.zeros((64, 32), dtype=torch.float16)), dict(idx=torch.zeros((63, 4), dtype=torch.int32)),
               dict(idx=torch.zeros((64, 3), dtype=torch.int32)), dict(idx=torch.zeros((64, 8), dtype=torch.int16)),
               dict(D=torch.zeros((64, 16)))):
        args = dict(Ac=Ac, idx=idx, B=Bs, D=D)
        args.update(kw)
        with pytest.raises(ValueError):
            mm.gemm_sparse24(args["Ac"], args["idx"], args["B"], args["D"], K=128)
    A16 = torch.zeros((64, 128), dtype=torch.float16)
    for Acx, idxx, badx in ((torch.zeros((64, 32), dtype=torch.float16), idx, None),
                            (Ac, torch.zeros((64, 3), dtype=torch.int32), None),
                            (Ac, idx, torch.zeros(0, dtype=torch.int32))):
        with pytest.raises(ValueError):
            mm.sparse24_compress(A16, Acx, idxx, badx)
        with pytest.raises(ValueError):
            mm.sparse24_prune_compress(A16, Acx, idxx, badx)


def static_dense(L, **kw):
    a = dict(a=mm.BF16, b=mm.BF16, M=64, N=64, K=64, alpha=1.0, A=P, lda=64, B=P, ldb=64, beta=0.0,
             C=None, ldc=64, D=P, ldd=64, ep=None, stream=None)
    a.update(kw)
    return L.mmac_gemm_dense_static(a["a"], a["b"], a["M"], a["N"], a["K"], a["alpha"], a["A"], a["lda"], a["B"],
                                    a["ldb"], a["beta"], a["C"], a["ldc"], a["D"], a["ldd"], a["ep"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(a=mm.BF16, b=mm.F16), mm.ERR_UNSUPPORTED),
    (dict(M=-1), mm.ERR_INVALID_ARG),
    (dict(A=None), mm.ERR_INVALID_ARG),
    (dict(beta=1.0, C=None), mm.ERR_INVALID_ARG),
    (dict(alpha=3.5e38), mm.ERR_INVALID_ARG),
    (dict(lda=68), mm.ERR_MISALIGNED),
    (dict(M=0), mm.OK),
])
def test_static_entry_validates_like_the_workspace_call(L, kw, code):
    assert static_dense(L, **kw) == code


def test_static_entry_rejects_plans_beyond_its_scratch(L, monkeypatch):
    """A forced plan larger than the fixed array is refused before any GPU work (the pointers here
    are fake, so a launch would fault); the library's own plans fit."""
    monkeypatch.setenv("MMAC_TILE", "256")
    monkeypatch.setenv("MMAC_SPLITK", "8")
    M, N, K = 1024, 1024, 65536                   # 16 tiles x 8 ranges x 256 KiB > 8 MiB
    assert mm.workspace_bytes(mm.BF16, M, N, K) > (8 << 20)
    assert static_dense(L, M=M, N=N, K=K, lda=K, ldb=K, ldd=N) == mm.ERR_SCRATCH
    monkeypatch.delenv("MMAC_TILE")
    monkeypatch.delenv("MMAC_SPLITK")
    worst = 0
    for M, N, K in ((64, 64, 1 << 20), (512, 512, 32768), (1024, 1024, 65536), (2048, 512, 65536),
                    (1000, 1000, 100000), (64, 8192, 65536)):
        for t in (mm.BF16, mm.I8, mm.FP8_E4M3):
            worst = max(worst, mm.workspace_bytes(t, M, N, K))
    assert 0 < worst <= (8 << 20)


def test_rate_library_exports_its_header():
    """libmmac_rate.so (the matrix-instruction rate microbenchmark) exports what include/mmac_rate.h
    declares, and its host-side queries answer without a GPU."""
    import ctypes
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "mmac_rate.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(mmac_rate_[a-z0-9_]+)\s*\(", text)))
    assert names == ["mmac_rate_name", "mmac_rate_ops", "mmac_rate_run", "mmac_rate_run_data", "mmac_rate_wall_clock_khz"]
    from sparse_matrix_multiply_amd import rate
    if not os.path.exists(rate.LIB_PATH):
        from sparse_matrix_multiply_amd import build
        build.build()
    L = rate.lib()
    for n in names:
        assert hasattr(L, n), n
    assert L.mmac_rate_ops(rate.MFMA_BF16) == 2 * 32 * 32 * 16
    assert L.mmac_rate_ops(rate.SMFMAC_FP8) == 2 * 32 * 32 * 64          # dense-equivalent K
    assert L.mmac_rate_ops(99) == 0 and L.mmac_rate_name(99) is None
    assert rate.name(rate.MFMA_FP8).startswith("v_mfma_scale_f32_32x32x64_f8f6f4")
    # argument errors return before any launch (fake pointers)
    assert L.mmac_rate_run(99, 1, 1, ctypes.c_void_p(P), ctypes.c_void_p(P), None) == -1
    assert L.mmac_rate_run(0, 0, 1, ctypes.c_void_p(P), ctypes.c_void_p(P), None) == -1
    assert L.mmac_rate_run_data(0, 2, 1, 1, ctypes.c_void_p(P), ctypes.c_void_p(P), None) == -1   # data flag 0 or 1
    assert L.mmac_rate_run_data(0, 1, 0, 1, ctypes.c_void_p(P), ctypes.c_void_p(P), None) == -1


def test_kernel_source_hash_ignores_comments_only():
    """The recorded counter traffic stays valid across comment edits and lapses on a code edit."""
    import bench
    code = 'int a = 1; // note\n/* block\n comment */ const char *s = "x // y /* z */";\nchar q = \'"\';  int  b;'
    assert bench._code_only(code) == 'int a = 1; const char *s = "x // y /* z */"; char q = \'"\'; int b;'
    assert bench._code_only(code) == bench._code_only(code.replace("// note", "// other words"))
    assert bench._code_only(code) != bench._code_only(code.replace("int a = 1", "int a = 2"))


HUGE = [(1 << 62), (1 << 62) + 16, (1 << 63) - 16]     # leading dimensions whose byte pitch overflows int64


@pytest.mark.parametrize("ld", HUGE)
def test_huge_leading_dimensions_are_rejected_without_overflow(L, ld):
    """A leading dimension so large that ld * element size overflows a 64-bit integer is refused
    with MMAC_ERR_UNSUPPORTED (the pitch limit is compared by division), on every entry point, before
    anything is launched (the pointers here are not device memory)."""
    U = mm.ERR_UNSUPPORTED
    for kw in (dict(lda=ld), dict(ldb=ld), dict(ldd=ld), dict(beta=1.0, C=P + 4096, ldc=ld, ldd=64)):
        assert dense(L, **kw) == U, kw
        assert static_dense(L, **kw) == U, kw
        assert dense_layout(L, **kw) == U, kw
    for kw in (dict(ldac=ld), dict(ldidx=ld), dict(ldb=ld), dict(ldd=ld)):
        assert sparse(L, **kw) == U, kw
    for entry in ("mmac_sparse24_compress", "mmac_sparse24_prune_compress"):
        for kw in (dict(lda=ld), dict(ldac=ld), dict(ldidx=ld)):
            assert compress(L, entry, **kw) == U, (entry, kw)
    for kw in (dict(lda=ld), dict(ldb=ld), dict(ldsa=ld), dict(ldsb=ld)):
        assert dense_mx(L, **kw) == U, kw


def test_compressor_pitch_limit(L):
    """The compressor takes the row-pitch limit of the other calls: 8 MiB for A and Ac, 2 Mi words
    for idx; one step past it is MMAC_ERR_UNSUPPORTED."""
    for entry in ("mmac_sparse24_compress", "mmac_sparse24_prune_compress"):
        assert compress(L, entry, lda=(1 << 22) + 8) == mm.ERR_UNSUPPORTED       # f16: 8 MiB + 16 bytes
        assert compress(L, entry, ldac=(1 << 22) + 8) == mm.ERR_UNSUPPORTED
        assert compress(L, entry, ldidx=(1 << 21) + 1) == mm.ERR_UNSUPPORTED
        assert compress(L, entry, a=mm.FP8_E4M3, lda=(1 << 23) + 16) == mm.ERR_UNSUPPORTED


def test_grid_count_limit(L):
    """An output so large that its tile count would overflow the 32-bit grid is refused (only a
    product of terabytes comes near it; the pointers here are not device memory)."""
    assert dense(L, M=(1 << 31) - 1, N=(1 << 21) - 64, K=16, lda=16, ldb=16, ldd=(1 << 21) - 64) == mm.ERR_UNSUPPORTED
