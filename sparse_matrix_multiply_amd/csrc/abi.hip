// C ABI of libmmac: argument validation on the host, kernel selection, launch
// on the caller's stream.  The public contract is in include/mmac.h.
#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>

#include "launch.h"
#include "mmac.h"

using namespace mmac;

namespace {

constexpr int64_t kMaxDim = 0x7fffffff;          // M, N, K below 2^31
constexpr int64_t kMaxPitchBytes = (int64_t)1 << 23;  // 256 rows of a tile must span < 2^31 bytes

int elem_size(int t) { return (t == MMAC_F16 || t == MMAC_BF16) ? 2 : 1; }
bool valid_type(int t) { return t >= MMAC_F16 && t <= MMAC_BF8_E5M2; }
bool is_fp8(int t) { return t == MMAC_FP8_E4M3 || t == MMAC_BF8_E5M2; }

bool supported_pair(int a, int b) {
    if (!valid_type(a) || !valid_type(b)) return false;
    if (is_fp8(a)) return is_fp8(b);
    return a == b;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

bool integral_i32(double v) { return std::isfinite(v) && v == std::floor(v) && v >= -2147483648.0 && v <= 2147483647.0; }

// Optional overrides for tuning: MMAC_TILE=256|2561|1282|128|64|16 (2561 = 256 x 128, 1282 = 128 x 256,
// 16 = skinny, M <= 32), MMAC_GROUP_M=<n>.
int env_int(const char *name, int dflt) {
    const char *s = std::getenv(name);
    if (!s || !*s) return dflt;
    return std::atoi(s);
}

TileShape pick_shape(int64_t M, int64_t N, bool sparse = false) {
    const int forced = env_int("MMAC_TILE", 0);
    if (forced == 256) return TILE_256;
    if (forced == 2561) return TILE_256x128;
    if (forced == 1282) return TILE_128x256;
    if (forced == 128) return TILE_128;
    if (forced == 64) return TILE_64;
    if (forced == 16 && !sparse && M <= 32) return TILE_SKINNY;
    // At most 32 rows: stream B once with the skinny kernel (dense A only).
    if (!sparse && M <= 32) return TILE_SKINNY;
    // Largest tile that still gives about one tile per compute unit (256 CUs).
    // Between 256 x 256 and 128 x 128 come the two 128 x 256 halves: 128 x 256
    // measured at least as fast on both 8192 x 1024 and 1024 x 8192 (K 8192),
    // so it wins unless 256 x 128 pads less (N below 256, say).
    auto tiles = [&](int tm, int tn) { return ((M + tm - 1) / tm) * ((N + tn - 1) / tn); };
    if (tiles(256, 256) >= 192) return TILE_256;
    const bool wide = tiles(128, 256) >= 192, tall = tiles(256, 128) >= 192;
    if (wide && (!tall || tiles(128, 256) <= tiles(256, 128))) return TILE_128x256;
    if (tall) return TILE_256x128;
    if (tiles(128, 128) >= 192) return TILE_128;
    return TILE_64;
}

// The epilogue variant a call asks for (NULL: the plain call).
mmac_epilogue_t epilogue_of(const mmac_epilogue_t *ep) {
    return ep ? *ep : mmac_epilogue_t{MMAC_OUT_ACC, MMAC_ACT_NONE, nullptr};
}

// Bytes of one C / D element.
int out_size(const mmac_epilogue_t &ep) {
    return ep.d_type == MMAC_OUT_ACC ? 4 : ep.d_type <= MMAC_OUT_F16 ? 2 : 1;
}

bool aligned_to(const void *p, int n) { return reinterpret_cast<uintptr_t>(p) % n == 0; }

// Common checks of the GEMM calls.  Returns MMAC_OK or the error.
mmac_status_t check_gemm(int a, int b, int64_t M, int64_t N, int64_t K, double alpha, const void *A,
                         int64_t lda, int64_t a_cols, const void *B, int64_t ldb, double beta, const void *C,
                         int64_t ldc, const void *D, int64_t ldd, const mmac_epilogue_t &ep, int64_t b_cols = -1) {
    if (b_cols < 0) b_cols = K;   // elements per memory row of B
    if (!supported_pair(a, b)) return MMAC_ERR_UNSUPPORTED;
    if (ep.d_type < MMAC_OUT_ACC || ep.d_type > MMAC_OUT_BF8_E5M2 || ep.act < MMAC_ACT_NONE || ep.act > MMAC_ACT_RELU)
        return MMAC_ERR_INVALID_ARG;
    if (a == MMAC_I8 && (ep.d_type != MMAC_OUT_ACC || ep.act != MMAC_ACT_NONE || ep.bias))
        return MMAC_ERR_UNSUPPORTED;
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return MMAC_ERR_INVALID_ARG;
    if ((K > 0 && (!A || !B)) || !D) return MMAC_ERR_INVALID_ARG;
    if (beta != 0.0 && !C) return MMAC_ERR_INVALID_ARG;
    if (lda < a_cols || ldb < b_cols || lda < 1 || ldb < 1 || ldd < N || (C && beta != 0.0 && ldc < N))
        return MMAC_ERR_INVALID_ARG;
    // alpha and beta are used in fp32 (the epilogue's precision): they must be finite there
    if (!std::isfinite(alpha) || !std::isfinite(beta) || std::fabs(alpha) > (double)FLT_MAX ||
        std::fabs(beta) > (double)FLT_MAX)
        return MMAC_ERR_INVALID_ARG;
    if (a == MMAC_I8 && (!integral_i32(alpha) || !integral_i32(beta))) return MMAC_ERR_INVALID_ARG;
    if (C == D && beta != 0.0 && ldc != ldd) return MMAC_ERR_INVALID_ARG;
    // pitch limits compared by division, so that no leading dimension, however large, overflows
    const int es = elem_size(a);
    if (lda > kMaxPitchBytes / es || ldb > kMaxPitchBytes / es) return MMAC_ERR_UNSUPPORTED;
    const int oes = out_size(ep);
    if (ldd > kMaxPitchBytes / oes || (C && beta != 0.0 && ldc > kMaxPitchBytes / oes)) return MMAC_ERR_UNSUPPORTED;
    // the grid (one workgroup per tile and K range) must fit a 32-bit count at the smallest tile
    // and the most ranges; only an output of terabytes comes near this
    if (((M + 63) / 64) * ((N + 63) / 64) > (int64_t)INT32_MAX / 8) return MMAC_ERR_UNSUPPORTED;
    if (!aligned16(A) || !aligned16(B) || (lda * es) % 16 || (ldb * es) % 16) return MMAC_ERR_MISALIGNED;
    if (!aligned_to(D, oes) || (C && beta != 0.0 && !aligned_to(C, oes))) return MMAC_ERR_MISALIGNED;
    if (ep.bias && !aligned4(ep.bias)) return MMAC_ERR_MISALIGNED;
    return MMAC_OK;
}

GemmParams make_params(int a, int64_t M, int64_t N, int64_t K, double alpha, const void *A, int64_t lda,
                       const void *B, int64_t ldb, double beta, const void *C, int64_t ldc, void *D, int64_t ldd,
                       const mmac_epilogue_t &ep, TileShape shape) {
    GemmParams p{};
    const int es = elem_size(a);
    p.A = static_cast<const uint8_t *>(A);
    p.a_pitch = lda * es;
    p.B = static_cast<const uint8_t *>(B);
    p.b_pitch = ldb * es;
    p.ldc = ldc;
    p.D = D;
    p.ldd = ldd;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.alpha = (float)alpha;
    p.beta = (float)beta;
    p.ialpha = a == MMAC_I8 ? (int)alpha : 0;
    p.ibeta = a == MMAC_I8 ? (int)beta : 0;
    // C is read only when beta is non-zero in the precision it is applied in
    p.use_c = (a == MMAC_I8 ? beta != 0.0 : p.beta != 0.0f) ? 1 : 0;
    p.C = p.use_c ? C : nullptr;
    if (p.use_c) {
        // beta * C folded into the accumulator's start value only where that adds no scaling of its
        // own: with alpha == 1 the start value is beta * C (the unfolded epilogue's product), with
        // alpha == beta it is C and the epilogue's alpha scales both terms.  Any other ratio would
        // start from (beta / alpha) * C, which can overflow or underflow fp32 while beta * C and
        // the result do not (alpha = 2^-100, beta = 2^100, say), so C is then read in the epilogue.
        if (a == MMAC_I8) {
            p.fold_c = alpha == 1.0;
        } else if (p.alpha == p.beta) {
            p.fold_c = 1;
            p.c_scale = 1.0f;
        } else if (p.alpha == 1.0f) {
            p.fold_c = 1;
            p.c_scale = p.beta;
        }
    }
    // C is folded into the accumulator only for fp32 / int32 outputs (16- and
    // 8-bit C is read in the epilogue)
    if (ep.d_type != MMAC_OUT_ACC) p.fold_c = 0;
    p.vec_d = aligned16(D) && (ldd * out_size(ep)) % 16 == 0;
    p.vec_c = p.use_c && aligned16(C) && (ldc * out_size(ep)) % 16 == 0;
    p.d_type = ep.d_type;
    p.act = ep.act;
    p.bias = ep.bias;
    const int tm = tile_rows(shape), tn = tile_cols(shape);
    p.tiles_m = (int)((M + tm - 1) / tm);
    p.tiles_n = (int)((N + tn - 1) / tn);
    p.group_m = std::max(1, env_int("MMAC_GROUP_M", 8));
    p.splits = 1;
    p.kt_per_split = 0x7fffffff;
    return p;
}

// ---- split-K -------------------------------------------------------------
// K elements per k-tile of the tiled kernels (16-bit elements: 64; 8-bit: 128).
int64_t k_tile(int a) { return elem_size(a) == 2 ? 64 : 128; }

struct SplitPlan {
    TileShape shape;
    int splits;
    int64_t kt_per_split;
    int64_t counter_bytes, bytes;   // workspace: counters, then the partial tiles
};

// Split-K when even the tile shape picked above leaves most of the 256
// compute units idle (at most 128 tiles) and K is long: S = 256 / tiles
// ranges (at most 8, each at least 8 k-tiles) of that shape.  Measured on
// MI355X: 512 x 512 x 32768 bf16 runs 2.1x faster with 4 ranges of 64 x 64
// tiles, 256 x 256 x 65536 3.3x with 4, 1024 x 512 x 8192 1.4x with 2; with
// about one tile per compute unit already (an 8192 x 1024 output in 128 x 256
// tiles) splitting only adds the partial-tile traffic.  MMAC_SPLITK=<S>
// forces S ranges.
SplitPlan plan_split(int a, int64_t M, int64_t N, int64_t K, bool sparse) {
    SplitPlan sp{pick_shape(M, N, sparse), 1, 0, 0, 0};
    if (sp.shape == TILE_SKINNY || M == 0 || N == 0 || K == 0) return sp;
    const int64_t nkt = (K + k_tile(a) - 1) / k_tile(a);
    const int64_t tm = tile_rows(sp.shape), tn = tile_cols(sp.shape);
    const int64_t tiles = ((M + tm - 1) / tm) * ((N + tn - 1) / tn);
    int64_t S = env_int("MMAC_SPLITK", 0);
    if (S <= 0) S = tiles <= 128 ? std::min<int64_t>({8, 256 / tiles, nkt / 8}) : 1;
    S = std::max<int64_t>(1, std::min<int64_t>(S, nkt));
    if (S < 2) return sp;
    sp.kt_per_split = (nkt + S - 1) / S;
    sp.splits = (int)((nkt + sp.kt_per_split - 1) / sp.kt_per_split);   // no empty range
    if (sp.splits < 2) return SplitPlan{sp.shape, 1, 0, 0, 0};
    sp.counter_bytes = (tiles * 4 + 255) / 256 * 256;
    sp.bytes = sp.counter_bytes + tiles * sp.splits * tm * tn * 4;
    return sp;
}

// Applies a split plan when the workspace holds it; otherwise the unsplit shape.
TileShape apply_split(GemmParams &p, const SplitPlan &sp, int64_t M, int64_t N, bool sparse, void *ws,
                      int64_t ws_bytes) {
    if (sp.splits < 2 || !ws || ws_bytes < sp.bytes) return pick_shape(M, N, sparse);
    p.splits = sp.splits;
    p.kt_per_split = (int)sp.kt_per_split;
    p.counters = static_cast<uint32_t *>(ws);
    p.partials = static_cast<uint8_t *>(ws) + sp.counter_bytes;
    const int tm = tile_rows(sp.shape), tn = tile_cols(sp.shape);
    p.tiles_m = (int)((M + tm - 1) / tm);
    p.tiles_n = (int)((N + tn - 1) / tn);
    return sp.shape;
}

mmac_status_t launched(hipError_t e) { return e == hipSuccess ? MMAC_OK : MMAC_ERR_HIP; }

// Shared by the plain and the pruning compressor.
mmac_status_t compress_call(mmac_dtype_t a_type, int64_t M, int64_t K, const void *A, int64_t lda, void *Ac,
                            int64_t ldac, uint32_t *idx, int64_t ldidx, uint32_t *bad_groups, bool prune,
                            void *stream) {
    if (!valid_type(a_type)) return MMAC_ERR_UNSUPPORTED;
    if (M < 0 || K < 0 || M > kMaxDim || K > kMaxDim || (K % 4) != 0) return MMAC_ERR_INVALID_ARG;
    if (!A || !Ac || !idx) return MMAC_ERR_INVALID_ARG;
    const int64_t words = (K + 31) / 32;
    if (lda < K || ldac < K / 2 || ldidx < words || lda < 1 || ldac < 1 || ldidx < 1) return MMAC_ERR_INVALID_ARG;
    const int es = elem_size(a_type);
    if (lda > kMaxPitchBytes / es || ldac > kMaxPitchBytes / es || ldidx > kMaxPitchBytes / 4)
        return MMAC_ERR_UNSUPPORTED;
    if (!aligned16(A) || !aligned16(Ac) || (lda * es) % 16 || (ldac * es) % 16) return MMAC_ERR_MISALIGNED;
    if (!aligned4(idx) || (bad_groups && !aligned4(bad_groups))) return MMAC_ERR_MISALIGNED;
    if (M == 0 || K == 0) return MMAC_OK;
    CompressParams p{};
    p.A = static_cast<const uint8_t *>(A);
    p.a_pitch = lda * es;
    p.Ac = static_cast<uint8_t *>(Ac);
    p.ac_pitch = ldac * es;
    p.idx = idx;
    p.idx_pitch = ldidx;
    p.bad = bad_groups;
    p.M = (int)M;
    p.K = (int)K;
    return launched(launch_compress(a_type, p, prune, static_cast<hipStream_t>(stream)));
}

// ---- the allocation-free split-K call ----------------------------------
// The split-K workspace of mmac_gemm_dense_static: one fixed array per GPU
// (tile counters first, then the partial tiles), held from the library's
// load until the process ends.  Host code never passes the array's name to a
// kernel or a copy: that is a host-side stand-in, not a device address.  It
// uses the address hipGetSymbolAddress gives for the current device.
constexpr int64_t kScratchBytes = MMAC_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ void zero_fill(uint4 *p, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = uint4{0u, 0u, 0u, 0u};
}

constexpr int kMaxDevices = 64;
struct DeviceScratch {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};
DeviceScratch g_scratch[kMaxDevices];

// This device's copy of `scratch`, set up once per device with that device
// current: its address (hipGetSymbolAddress, return code checked) and one
// fill kernel on `stream` that zeroes it, since the tile counters must start
// at zero (every complete call leaves them zero again).  A fill kernel, not a
// memset, so that a call captured into a HIP graph records only kernels.
// Returns NULL (and the error) if the address cannot be had.
void *device_scratch(hipStream_t stream, hipError_t *err) {
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    DeviceScratch &d = g_scratch[dev];
    std::call_once(d.once, [&] {
        void *ptr = nullptr;
        d.err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (d.err == hipSuccess) {
            hipLaunchKernelGGL(zero_fill, dim3(256), dim3(256), 0, stream, static_cast<uint4 *>(ptr),
                               kScratchBytes / 16);
            d.err = hipGetLastError();
        }
        if (d.err == hipSuccess) d.ptr = ptr;
    });
    *err = d.err;
    return d.ptr;
}

}  // namespace

extern "C" {

mmac_status_t mmac_gemm_dense_static(mmac_dtype_t a_type, mmac_dtype_t b_type, int64_t M, int64_t N, int64_t K,
                                     double alpha, const void *A, int64_t lda, const void *B, int64_t ldb,
                                     double beta, const void *C, int64_t ldc, void *D, int64_t ldd,
                                     const mmac_epilogue_t *ep_in, void *stream) {
    const mmac_epilogue_t ep = epilogue_of(ep_in);
    const mmac_status_t st = check_gemm(a_type, b_type, M, N, K, alpha, A, lda, K, B, ldb, beta, C, ldc, D, ldd, ep);
    if (st != MMAC_OK) return st;
    if (M == 0 || N == 0) return MMAC_OK;
    const int64_t need = pick_shape(M, N) == TILE_SKINNY ? 0 : plan_split(a_type, M, N, K, false).bytes;
    if (need > kScratchBytes) return MMAC_ERR_SCRATCH;
    void *ws = nullptr;
    if (need > 0) {
        hipError_t e;
        ws = device_scratch(static_cast<hipStream_t>(stream), &e);
        if (!ws) return MMAC_ERR_HIP;
    }
    return mmac_gemm_dense_ws(a_type, b_type, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, D, ldd, ep_in, ws,
                              ws ? kScratchBytes : 0, stream);
}

mmac_status_t mmac_gemm_dense_ws(mmac_dtype_t a_type, mmac_dtype_t b_type, int64_t M, int64_t N, int64_t K,
                                 double alpha, const void *A, int64_t lda, const void *B, int64_t ldb, double beta,
                                 const void *C, int64_t ldc, void *D, int64_t ldd, const mmac_epilogue_t *ep_in,
                                 void *workspace, int64_t workspace_bytes, void *stream) {
    const mmac_epilogue_t ep = epilogue_of(ep_in);
    const mmac_status_t st = check_gemm(a_type, b_type, M, N, K, alpha, A, lda, K, B, ldb, beta, C, ldc, D, ldd, ep);
    if (st != MMAC_OK) return st;
    if (workspace_bytes < 0) return MMAC_ERR_INVALID_ARG;
    if (workspace && !aligned16(workspace)) return MMAC_ERR_MISALIGNED;
    if (M == 0 || N == 0) return MMAC_OK;
    TileShape shape = pick_shape(M, N);
    GemmParams p = make_params(a_type, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, D, ldd, ep, shape);
    if (shape == TILE_SKINNY)
        return launched(launch_gemm_skinny(a_type, b_type, p, static_cast<hipStream_t>(stream)));
    shape = apply_split(p, plan_split(a_type, M, N, K, false), M, N, false, workspace, workspace_bytes);
    return launched(launch_gemm_dense(a_type, b_type, shape, p, static_cast<hipStream_t>(stream)));
}

mmac_status_t mmac_gemm_dense_ep(mmac_dtype_t a_type, mmac_dtype_t b_type, int64_t M, int64_t N, int64_t K,
                                 double alpha, const void *A, int64_t lda, const void *B, int64_t ldb, double beta,
                                 const void *C, int64_t ldc, void *D, int64_t ldd, const mmac_epilogue_t *ep,
                                 void *stream) {
    return mmac_gemm_dense_ws(a_type, b_type, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, D, ldd, ep, nullptr, 0,
                              stream);
}

mmac_status_t mmac_gemm_dense(mmac_dtype_t a_type, mmac_dtype_t b_type, int64_t M, int64_t N, int64_t K,
                              double alpha, const void *A, int64_t lda, const void *B, int64_t ldb, double beta,
                              const void *C, int64_t ldc, void *D, int64_t ldd, void *stream) {
    return mmac_gemm_dense_ep(a_type, b_type, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, D, ldd, nullptr, stream);
}

mmac_status_t mmac_sparse24_compress(mmac_dtype_t a_type, int64_t M, int64_t K, const void *A, int64_t lda,
                                     void *Ac, int64_t ldac, uint32_t *idx, int64_t ldidx, uint32_t *bad_groups,
                                     void *stream) {
    return compress_call(a_type, M, K, A, lda, Ac, ldac, idx, ldidx, bad_groups, false, stream);
}

mmac_status_t mmac_sparse24_prune_compress(mmac_dtype_t a_type, int64_t M, int64_t K, const void *A, int64_t lda,
                                           void *Ac, int64_t ldac, uint32_t *idx, int64_t ldidx,
                                           uint32_t *bad_groups, void *stream) {
    return compress_call(a_type, M, K, A, lda, Ac, ldac, idx, ldidx, bad_groups, true, stream);
}

mmac_status_t mmac_gemm_sparse24_ws(mmac_dtype_t a_type, mmac_dtype_t b_type, int64_t M, int64_t N, int64_t K,
                                    double alpha, const void *Ac, int64_t ldac, const uint32_t *idx, int64_t ldidx,
                                    const void *B, int64_t ldb, double beta, const void *C, int64_t ldc, void *D,
                                    int64_t ldd, const mmac_epilogue_t *ep_in, void *workspace,
                                    int64_t workspace_bytes, void *stream) {
    const mmac_epilogue_t ep = epilogue_of(ep_in);
    if (K >= 0 && (K % 4) != 0) return MMAC_ERR_INVALID_ARG;
    const mmac_status_t st =
        check_gemm(a_type, b_type, M, N, K, alpha, Ac, ldac, K / 2, B, ldb, beta, C, ldc, D, ldd, ep);
    if (st != MMAC_OK) return st;
    if ((K > 0 && !idx) || ldidx < (K + 31) / 32 || ldidx < 1) return MMAC_ERR_INVALID_ARG;
    if (ldidx > kMaxPitchBytes / 4) return MMAC_ERR_UNSUPPORTED;   // 256 rows of index words below 2^31 bytes
    if (!aligned4(idx)) return MMAC_ERR_MISALIGNED;
    if (workspace_bytes < 0) return MMAC_ERR_INVALID_ARG;
    if (workspace && !aligned16(workspace)) return MMAC_ERR_MISALIGNED;
    if (M == 0 || N == 0) return MMAC_OK;
    GemmParams p = make_params(a_type, M, N, K, alpha, Ac, ldac, B, ldb, beta, C, ldc, D, ldd, ep,
                               pick_shape(M, N, true));
    p.idx = idx;
    p.idx_pitch = ldidx;
    const TileShape shape =
        apply_split(p, plan_split(a_type, M, N, K, true), M, N, true, workspace, workspace_bytes);
    return launched(launch_gemm_sparse(a_type, b_type, shape, p, static_cast<hipStream_t>(stream)));
}

mmac_status_t mmac_gemm_sparse24_ep(mmac_dtype_t a_type, mmac_dtype_t b_type, int64_t M, int64_t N, int64_t K,
                                    double alpha, const void *Ac, int64_t ldac, const uint32_t *idx, int64_t ldidx,
                                    const void *B, int64_t ldb, double beta, const void *C, int64_t ldc, void *D,
                                    int64_t ldd, const mmac_epilogue_t *ep, void *stream) {
    return mmac_gemm_sparse24_ws(a_type, b_type, M, N, K, alpha, Ac, ldac, idx, ldidx, B, ldb, beta, C, ldc, D, ldd,
                                 ep, nullptr, 0, stream);
}

mmac_status_t mmac_gemm_dense_mx(mmac_dtype_t a_type, mmac_dtype_t b_type, int64_t M, int64_t N, int64_t K,
                                 double alpha, const void *A, int64_t lda, const uint32_t *SA, int64_t ldsa,
                                 const void *B, int64_t ldb, const uint32_t *SB, int64_t ldsb, double beta,
                                 const void *C, int64_t ldc, void *D, int64_t ldd, const mmac_epilogue_t *ep_in,
                                 void *stream) {
    const mmac_epilogue_t ep = epilogue_of(ep_in);
    // FP4 (packed two per byte) only with FP4, FP6 (four per three bytes) only
    // with FP6; the generic checks below then see them as a one-byte type with
    // the rows' byte counts
    const bool fp4 = a_type == MMAC_FP4_E2M1 || b_type == MMAC_FP4_E2M1;
    const bool fp6a = a_type == MMAC_FP6_E2M3 || a_type == MMAC_BF6_E3M2;
    const bool fp6b = b_type == MMAC_FP6_E2M3 || b_type == MMAC_BF6_E3M2;
    const bool fp6 = fp6a || fp6b, packed = fp4 || fp6;
    if (fp4 && a_type != b_type) return MMAC_ERR_UNSUPPORTED;
    if (fp6 && !(fp6a && fp6b)) return MMAC_ERR_UNSUPPORTED;
    if (!packed && valid_type(a_type) && valid_type(b_type) && (!is_fp8(a_type) || !is_fp8(b_type)))
        return MMAC_ERR_UNSUPPORTED;
    if (K >= 0 && (K % 32) != 0) return MMAC_ERR_INVALID_ARG;
    if (fp4 && ((lda % 2) || (ldb % 2))) return MMAC_ERR_MISALIGNED;
    if (fp6 && ((lda % 4) || (ldb % 4))) return MMAC_ERR_MISALIGNED;
    const auto bytes = [&](int64_t n) { return fp4 ? n / 2 : fp6 ? n / 4 * 3 : n; };   // of n elements
    const mmac_dtype_t ga = packed ? MMAC_FP8_E4M3 : a_type, gb = packed ? MMAC_FP8_E4M3 : b_type;
    const int64_t kk = bytes(K);
    const mmac_status_t st =
        check_gemm(ga, gb, M, N, kk, alpha, A, bytes(lda), kk, B, bytes(ldb), beta, C, ldc, D, ldd, ep);
    if (st != MMAC_OK) return st;
    if ((K > 0 && (!SA || !SB)) || ldsa < M || ldsb < N || ldsa < 1 || ldsb < 1) return MMAC_ERR_INVALID_ARG;
    const int64_t scale_rows = (K + 127) / 128;
    // scale arrays of scale_rows rows of ld words below 2^31 bytes (compared by division: no overflow)
    if (scale_rows > 0 && std::max(ldsa, ldsb) > ((((int64_t)1 << 31) - 1) / 4) / scale_rows)
        return MMAC_ERR_UNSUPPORTED;
    if ((ldsa % 4) || (ldsb % 4) || !aligned16(SA) || !aligned16(SB)) return MMAC_ERR_MISALIGNED;
    if (M == 0 || N == 0) return MMAC_OK;
    // the 8-wave 256 x 256 tile has no registers left for the scale words: its 128 x 256 half instead
    TileShape shape = pick_shape(M, N, true);
    if (shape == TILE_256) shape = TILE_128x256;
    GemmParams p = make_params(ga, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, D, ldd, ep, shape);
    if (packed) {
        p.a_pitch = bytes(lda);
        p.b_pitch = bytes(ldb);
    }
    p.sa = SA;
    p.sb = SB;
    p.ldsa = ldsa;
    p.ldsb = ldsb;
    p.scale_rows = (int)scale_rows;
    return launched(launch_gemm_mx(a_type, b_type, shape, p, static_cast<hipStream_t>(stream)));
}

mmac_status_t mmac_gemm_dense_layout(mmac_dtype_t a_type, mmac_dtype_t b_type, int trans_a, int trans_b, int64_t M,
                                     int64_t N, int64_t K, double alpha, const void *A, int64_t lda, const void *B,
                                     int64_t ldb, double beta, const void *C, int64_t ldc, void *D, int64_t ldd,
                                     const mmac_epilogue_t *ep_in, void *stream) {
    if ((trans_a != 0 && trans_a != 1) || (trans_b != 0 && trans_b != 1)) return MMAC_ERR_INVALID_ARG;
    if (!trans_a && !trans_b)
        return mmac_gemm_dense_ep(a_type, b_type, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, D, ldd, ep_in, stream);
    const mmac_epilogue_t ep = epilogue_of(ep_in);
    const mmac_status_t st = check_gemm(a_type, b_type, M, N, K, alpha, A, lda, trans_a ? M : K, B, ldb, beta, C, ldc,
                                        D, ldd, ep, trans_b ? N : K);
    if (st != MMAC_OK) return st;
    // a transposed operand is addressed with one buffer over all its K rows
    const int64_t es = elem_size(a_type);
    if ((trans_a && K * lda * es >= ((int64_t)1 << 31)) || (trans_b && K * ldb * es >= ((int64_t)1 << 31)))
        return MMAC_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return MMAC_OK;
    const TileShape shape = pick_shape(M, N, true);
    const GemmParams p = make_params(a_type, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, D, ldd, ep, shape);
    return launched(
        launch_gemm_layout(a_type, b_type, trans_a != 0, trans_b != 0, shape, p, static_cast<hipStream_t>(stream)));
}

int64_t mmac_gemm_workspace_bytes(mmac_dtype_t a_type, int64_t M, int64_t N, int64_t K, int sparse) {
    if (!valid_type(a_type) || M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return 0;
    return plan_split(a_type, M, N, K, sparse != 0).bytes;
}

mmac_status_t mmac_gemm_sparse24(mmac_dtype_t a_type, mmac_dtype_t b_type, int64_t M, int64_t N, int64_t K,
                                 double alpha, const void *Ac, int64_t ldac, const uint32_t *idx, int64_t ldidx,
                                 const void *B, int64_t ldb, double beta, const void *C, int64_t ldc, void *D,
                                 int64_t ldd, void *stream) {
    return mmac_gemm_sparse24_ep(a_type, b_type, M, N, K, alpha, Ac, ldac, idx, ldidx, B, ldb, beta, C, ldc, D, ldd,
                                 nullptr, stream);
}

const char *mmac_status_string(mmac_status_t s) {
    switch (s) {
    case MMAC_OK: return "MMAC_OK";
    case MMAC_ERR_INVALID_ARG: return "MMAC_ERR_INVALID_ARG: invalid argument";
    case MMAC_ERR_UNSUPPORTED: return "MMAC_ERR_UNSUPPORTED: unsupported element types or sizes";
    case MMAC_ERR_MISALIGNED: return "MMAC_ERR_MISALIGNED: pointer or row pitch not aligned as required";
    case MMAC_ERR_HIP: return "MMAC_ERR_HIP: the HIP runtime refused the launch";
    case MMAC_ERR_SCRATCH:
        return "MMAC_ERR_SCRATCH: the split-K plan needs more than the library's fixed scratch array (8 MiB)";
    default: return "unknown mmac status";
    }
}

}  // extern "C"
