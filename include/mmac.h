/*
 * mmac -- tiled matrix multiply-accumulate on AMD Instinct MI355X (gfx950).
 *
 * Computes D = alpha * A*B + beta * C on one GPU, with A either dense or 4:2
 * structured-sparse (stored as its non-zeros plus a per-group index), using
 * the gfx950 dense MFMA and sparse SMFMAC matrix instructions.
 *
 * Operation (ROCm handbook, "CDNA dense MFMA builtins", section "Naming
 * convention"): a matrix instruction adds the contribution of a K-wide panel of
 * A (M x K) and of B (K x N) to an M x N tile of C, and the caller loops over K
 * to form the full product.  Each call below is that full product over a whole
 * matrix, scaled by alpha, plus beta * C.
 *
 * Sparse form ("CDNA3 sparse MFMA builtins", section "Structured sparsity (4:2
 * pattern)"): in every contiguous group of four elements of A along K at most
 * two are non-zero; the compressed A stores the two kept values of each group
 * in ascending position, half the K length, and the index gives their
 * positions p0 < p1 as the nibble p0 | (p1 << 2) (keeping positions {0,2} of a
 * group gives 0x8, as the page's 0x88 / 0x8888 examples show).
 *
 * Conventions shared by every call
 *   - Element types: see mmac_dtype_t.  FP8 and BF8 use the OCP encodings
 *     (E4M3 and E5M2), which gfx950 uses ("CDNA3 sparse MFMA builtins", note
 *     under "FP8 16x16 sparse kernel").
 *   - Layouts (all strides in elements):
 *       A   row-major    M x K :  A[i*lda + k],   lda >= K
 *       B   column-major K x N :  B[j*ldb + k],   ldb >= K
 *       C,D row-major    M x N :  D[i*ldd + j],   ldd >= N (ldc >= N)
 *       Ac  row-major    M x K/2: compressed A, ldac >= K/2
 *       idx row-major    M x ceil(K/32) 32-bit words, ldidx >= ceil(K/32);
 *           group g of row i (elements 4g..4g+3) is the nibble at bits
 *           4*(g mod 8) of word g/8; bits of groups at or past K/4 are zero.
 *   - Output type: float (fp32) for floating inputs, int32 for int8 inputs;
 *     C has the output type.  Floating results are accumulated in fp32; int8
 *     results are exact modulo 2^32 (two's complement wrap, no saturation).
 *   - beta == 0 means C is not read (C may be NULL; NaNs in C do not leak).
 *     D may be the same buffer as C when ldd == ldc; other overlaps between
 *     outputs and inputs are not allowed.
 *   - Floating inputs: alpha and beta are applied in fp32 (rounded to
 *     nearest from the double given); a value that is not finite or whose
 *     magnitude exceeds FLT_MAX (3.40282347e38) is MMAC_ERR_INVALID_ARG, and a
 *     beta that rounds to zero in fp32 reads no C.  beta * C enters the fp32
 *     sum unscaled by any ratio beta / alpha, so every finite pair of scales
 *     is exact to fp32 rounding (alpha = 2^-100 with beta = 2^100 included).
 *   - int8: alpha and beta must be integers that fit in int32.
 *   - M == 0 or N == 0: nothing is done.  K == 0: D = beta * C (A, B, Ac and
 *     idx are not read and may be NULL).
 *   - Alignment: A, B, Ac must start on a 16-byte boundary and their row
 *     pitch in bytes (ld * element size) must be a multiple of 16.  C, D and
 *     idx need only their natural 4-byte alignment.
 *   - Sizes: M, N, K must be below 2^31 (MMAC_ERR_INVALID_ARG otherwise); the
 *     row pitch of A, B, Ac, C and D must be at most 8 MiB and that of idx
 *     at most 8 MiB / 4 words (MMAC_ERR_UNSUPPORTED otherwise).
 *   - Memory: every pointer is device memory on the current HIP device, owned
 *     by the caller; the library never allocates, frees or keeps a pointer
 *     (its only device memory of its own is mmac_gemm_dense_static's array).
 *     Buffers must stay valid until the work on `stream` has finished.
 *   - Asynchrony: each call validates its arguments on the host, then enqueues
 *     kernels on `stream` (a hipStream_t of the current device; NULL is the
 *     default stream) and returns without synchronising.  A kernel fault shows up at the caller's
 *     next synchronisation.
 *   - Errors: no exception crosses this interface.  Argument errors are
 *     detected before any GPU work is enqueued; nothing is written then.
 *   - Thread safety: calls are re-entrant; the library keeps no state between
 *     calls (except mmac_gemm_dense_static's fixed scratch array, see there).
 *   - Tuning: two environment variables, read on every call, override the
 *     tile choice: MMAC_TILE (256, 128 or 64 forces that square output tile,
 *     2561 forces 256 x 128 and 1282 forces 128 x 256; 16 forces the
 *     one-wave-column path for M <= 32) and MMAC_GROUP_M (tile rows
 *     visited together by the scheduler, default 8).  Results do not depend
 *     on them beyond floating-point rounding.
 */
#ifndef MMAC_H
#define MMAC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MMAC_OK = 0,
    MMAC_ERR_INVALID_ARG = 1, /* negative or oversized dims, bad ld, NULL pointer, bad alpha/beta */
    MMAC_ERR_UNSUPPORTED = 2, /* element-type pair not supported */
    MMAC_ERR_MISALIGNED = 3,  /* alignment rule above broken */
    MMAC_ERR_HIP = 4,         /* the HIP runtime refused the launch */
    MMAC_ERR_SCRATCH = 5      /* mmac_gemm_dense_static: more scratch needed than its fixed array holds */
} mmac_status_t;

typedef enum {
    MMAC_F16 = 1,      /* IEEE binary16 */
    MMAC_BF16 = 2,     /* bfloat16 */
    MMAC_I8 = 3,       /* signed 8-bit integer */
    MMAC_FP8_E4M3 = 4, /* OCP FP8 E4M3 */
    MMAC_BF8_E5M2 = 5, /* OCP BF8 E5M2 */
    MMAC_FP4_E2M1 = 6, /* OCP FP4 E2M1, two per byte (element 2m in the low nibble of byte m);
                          block-scaled GEMM only */
    MMAC_FP6_E2M3 = 7, /* OCP FP6 E2M3 and BF6 E3M2, four elements per three bytes: element n of */
    MMAC_BF6_E3M2 = 8  /* a row in bits 6n .. 6n+5 of the row read as a little-endian bit string
                          (bit b = bit b mod 8 of byte b / 8); block-scaled GEMM only */
} mmac_dtype_t;

/*
 * Dense GEMM: D = alpha * A*B + beta * C.
 * Supported (a_type, b_type): (F16, F16), (BF16, BF16), (I8, I8), and every
 * pair of FP8_E4M3 / BF8_E5M2 (the page "CDNA3 sparse MFMA builtins" lists all
 * four FP8 x BF8 combinations).  Other pairs return MMAC_ERR_UNSUPPORTED.
 */
mmac_status_t mmac_gemm_dense(mmac_dtype_t a_type, mmac_dtype_t b_type,
                              int64_t M, int64_t N, int64_t K, double alpha,
                              const void *A, int64_t lda,
                              const void *B, int64_t ldb,
                              double beta, const void *C, int64_t ldc,
                              void *D, int64_t ldd, void *stream);

/*
 * 4:2 compression of a dense A ("CDNA3 sparse MFMA builtins", "Structured
 * sparsity (4:2 pattern)": walk K in groups of four and pack the two non-zeros
 * of each group one after the other).
 *   A    dense row-major M x K of a_type (any of the five types), K % 4 == 0.
 *   Ac   output, row-major M x K/2 of a_type.
 *   idx  output, row-major M x ceil(K/32) words (layout above).
 *   bad_groups  device pointer to one uint32 or NULL; if given, the number of
 *        groups with more than two non-zeros is atomically added to it (the
 *        caller clears it).
 * Rules per group: a non-zero is any element other than +0/-0 (floating) or 0
 * (int8); a NaN counts as non-zero.  More than two non-zeros: the two lowest
 * positions are kept and the group is counted in bad_groups.  Fewer than two:
 * the lowest unused positions fill the pair (their stored value is the zero
 * found there, bit for bit).  The output is bit-exact and deterministic.
 */
mmac_status_t mmac_sparse24_compress(mmac_dtype_t a_type, int64_t M, int64_t K,
                                     const void *A, int64_t lda,
                                     void *Ac, int64_t ldac,
                                     uint32_t *idx, int64_t ldidx,
                                     uint32_t *bad_groups, void *stream);

/*
 * Magnitude pruning to the 4:2 pattern fused with the compression above, in
 * one pass over A.  The pages give the pattern and the compressed form
 * ("CDNA3 sparse MFMA builtins", "Structured sparsity (4:2 pattern)") but not
 * how a dense A is brought to it; this keeps, in every group of four along K,
 * the two elements of largest magnitude:
 *   - |a| of the decoded value; int8 -128 has magnitude 128;
 *   - a NaN is larger than every number (infinities included), all NaNs tie;
 *   - ties go to the lower position.
 * The kept pair is stored as the compressor stores it (ascending positions,
 * bits copied, same index layout).  Arguments, alignment, error behaviour and
 * bad_groups (groups that held more than two non-zeros, i.e. the groups that
 * pruning changed) are those of mmac_sparse24_compress.  Output is bit-exact
 * and deterministic; on an A that already has the 4:2 pattern it equals the
 * plain compressor's.
 */
mmac_status_t mmac_sparse24_prune_compress(mmac_dtype_t a_type, int64_t M, int64_t K,
                                           const void *A, int64_t lda,
                                           void *Ac, int64_t ldac,
                                           uint32_t *idx, int64_t ldidx,
                                           uint32_t *bad_groups, void *stream);

/*
 * Sparse GEMM with a compressed 4:2 A: D = alpha * A*B + beta * C, where A is
 * the dense M x K matrix described by (Ac, idx) and B, C, D are as in
 * mmac_gemm_dense.  K is the dense K and must be a multiple of 4.  Supported
 * pairs are those of mmac_gemm_dense.  Every index nibble must name a pair
 * p0 < p1 (the compressor only writes such nibbles); other nibble values give
 * unspecified results.  Floating work is counted with the dense K
 * ("dense-equivalent": 2*M*N*K), as the page's sparse instruction table does.
 */
mmac_status_t mmac_gemm_sparse24(mmac_dtype_t a_type, mmac_dtype_t b_type,
                                 int64_t M, int64_t N, int64_t K, double alpha,
                                 const void *Ac, int64_t ldac,
                                 const uint32_t *idx, int64_t ldidx,
                                 const void *B, int64_t ldb,
                                 double beta, const void *C, int64_t ldc,
                                 void *D, int64_t ldd, void *stream);

/*
 * Epilogue variants ("Epilogue variants" below): the type of C and D, a
 * per-column bias and an activation, applied after alpha * A*B + beta * C.
 */
typedef enum {
    MMAC_OUT_ACC = 0,  /* fp32 (int32 for int8 inputs): the plain calls' output */
    MMAC_OUT_BF16 = 1, /* bfloat16 */
    MMAC_OUT_F16 = 2,  /* IEEE binary16 */
    MMAC_OUT_FP8_E4M3 = 3, /* OCP FP8 E4M3: largest finite 448, no infinities */
    MMAC_OUT_BF8_E5M2 = 4  /* OCP BF8 E5M2: largest finite 57344 */
} mmac_out_type_t;

typedef enum {
    MMAC_ACT_NONE = 0,
    MMAC_ACT_RELU = 1 /* max(v, 0): negative values become +0; NaN and -0 pass unchanged */
} mmac_act_t;

typedef struct mmac_epilogue {
    int32_t d_type;     /* mmac_out_type_t: element type of D and of C */
    int32_t act;        /* mmac_act_t */
    const float *bias;  /* NULL, or device memory holding N fp32 values (4-byte aligned) */
} mmac_epilogue_t;

/*
 * Epilogue variants of the two GEMMs.  Arguments are those of mmac_gemm_dense
 * and mmac_gemm_sparse24 plus `ep` (host pointer, read during the call only;
 * NULL means { MMAC_OUT_ACC, MMAC_ACT_NONE, NULL }, i.e. the plain call).
 * Every element of D is
 *     D[i][j] = round( act( alpha * acc[i][j] + beta * C[i][j] + bias[j] ) )
 * where acc is A*B accumulated in fp32, the sum is formed in fp32 (bias is
 * added only when given), and round converts to d_type: to nearest, ties to
 * even, saturating -- a finite value beyond the type's largest finite value
 * (bfloat16 0x7f7f, binary16 65504, E4M3 448, E5M2 57344) becomes that value
 * with its sign; infinities stay infinite (E4M3 has none: they saturate too);
 * NaN becomes the type's quiet NaN (0x7fc0, 0x7e00, 0x7f, 0x7e) with its
 * sign.  The fp8 encodings are the OCP ones gfx950 uses ("CDNA3 sparse MFMA
 * builtins", note under "FP8 16x16 sparse kernel").  C has d_type and row
 * pitch ldc; D has d_type and row pitch ldd.  16-bit C and D need 2-byte
 * alignment (8-bit: none), and the row pitch limit of 8 MiB applies to
 * ldc / ldd times the element size.
 * int8 inputs accept only { MMAC_OUT_ACC, MMAC_ACT_NONE, NULL }
 * (MMAC_ERR_UNSUPPORTED otherwise).  An unknown d_type or act gives
 * MMAC_ERR_INVALID_ARG; a bias not 4-byte aligned gives MMAC_ERR_MISALIGNED.
 * The pages define the product and the beta * C term only; the other steps
 * are the usual fused output stage of a GEMM library.
 */
mmac_status_t mmac_gemm_dense_ep(mmac_dtype_t a_type, mmac_dtype_t b_type,
                                 int64_t M, int64_t N, int64_t K, double alpha,
                                 const void *A, int64_t lda,
                                 const void *B, int64_t ldb,
                                 double beta, const void *C, int64_t ldc,
                                 void *D, int64_t ldd,
                                 const mmac_epilogue_t *ep, void *stream);

mmac_status_t mmac_gemm_sparse24_ep(mmac_dtype_t a_type, mmac_dtype_t b_type,
                                    int64_t M, int64_t N, int64_t K, double alpha,
                                    const void *Ac, int64_t ldac,
                                    const uint32_t *idx, int64_t ldidx,
                                    const void *B, int64_t ldb,
                                    double beta, const void *C, int64_t ldc,
                                    void *D, int64_t ldd,
                                    const mmac_epilogue_t *ep, void *stream);

/*
 * Split-K variants: the calls above, plus a caller-provided workspace that lets
 * the library cut K into up to four ranges when the output has too few
 * 256 x 256 tiles to occupy the GPU's 256 compute units (for example one
 * GPU's 8192 x 1024 share of an 8192^3 product).  Each (tile, K range) is one
 * workgroup; the range that finishes a tile last sums the fp32 (int32)
 * partial tiles in range order 0, 1, 2, ... and applies the epilogue, so
 * results are deterministic and independent of timing.
 *   workspace        device memory, 16-byte aligned, or NULL.  Its first
 *                    bytes hold one counter per output tile: they must be
 *                    zero before the first call that uses the workspace, and
 *                    every call leaves them zero again (zero it once after
 *                    allocating it, e.g. with hipMemset).
 *   workspace_bytes  its size.  If it is smaller than
 *                    mmac_gemm_workspace_bytes(...) for the call (or
 *                    workspace is NULL) the call runs unsplit, exactly as
 *                    the _ep call.  A negative size is MMAC_ERR_INVALID_ARG;
 *                    a misaligned workspace MMAC_ERR_MISALIGNED.
 * Calls that share a workspace must not run concurrently (different streams)
 * on the same device; calls in one stream may share it.  Results of a split
 * call differ from the unsplit call only by floating-point summation order
 * (int8: not at all).  MMAC_SPLITK=<S> in the environment forces S ranges
 * (if the workspace holds them).
 */
mmac_status_t mmac_gemm_dense_ws(mmac_dtype_t a_type, mmac_dtype_t b_type,
                                 int64_t M, int64_t N, int64_t K, double alpha,
                                 const void *A, int64_t lda,
                                 const void *B, int64_t ldb,
                                 double beta, const void *C, int64_t ldc,
                                 void *D, int64_t ldd, const mmac_epilogue_t *ep,
                                 void *workspace, int64_t workspace_bytes, void *stream);

mmac_status_t mmac_gemm_sparse24_ws(mmac_dtype_t a_type, mmac_dtype_t b_type,
                                    int64_t M, int64_t N, int64_t K, double alpha,
                                    const void *Ac, int64_t ldac,
                                    const uint32_t *idx, int64_t ldidx,
                                    const void *B, int64_t ldb,
                                    double beta, const void *C, int64_t ldc,
                                    void *D, int64_t ldd, const mmac_epilogue_t *ep,
                                    void *workspace, int64_t workspace_bytes, void *stream);

/*
 * Allocation-free split-K dense GEMM, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The same operation, arguments, rules and kernels as
 * mmac_gemm_dense_ws, except that the split-K workspace is the library's own
 * fixed device array of MMAC_STATIC_SCRATCH_BYTES (8 MiB): one copy per GPU,
 * created when the library is loaded and held until the process ends.  The
 * call allocates nothing and frees nothing.
 *   - The first call on a device looks up that device's copy and enqueues one
 *     small kernel on `stream` that zeroes it (the tile counters must start at
 *     zero; every complete call leaves them zero again).
 *   - A product whose split-K plan needs more than the array holds (only
 *     possible when MMAC_TILE / MMAC_SPLITK force a large plan; every plan the
 *     library picks by itself needs at most 4 MiB) returns MMAC_ERR_SCRATCH
 *     before any GPU work; a product that does not split uses no scratch.
 *   - All calls on one GPU share its array: calls that may overlap in time on
 *     one GPU (different streams, or different host threads without ordering)
 *     race on it and give undefined results.  Calls in one stream are safe.
 */
#define MMAC_STATIC_SCRATCH_BYTES (8 << 20)
mmac_status_t mmac_gemm_dense_static(mmac_dtype_t a_type, mmac_dtype_t b_type,
                                     int64_t M, int64_t N, int64_t K, double alpha,
                                     const void *A, int64_t lda,
                                     const void *B, int64_t ldb,
                                     double beta, const void *C, int64_t ldc,
                                     void *D, int64_t ldd, const mmac_epilogue_t *ep, void *stream);

/*
 * Block-scaled (MX) dense GEMM -- beyond the pages, which have no block
 * scales; the format is the OCP Microscaling one: along K, every block of 32
 * consecutive elements of a row of A (and of a column of B) shares one E8M0
 * scale, an unsigned exponent e with value 2^(e - 127).  Computes
 *   D = alpha * sum_b 2^(sa[i][b] - 127) * 2^(sb[j][b] - 127) * (A_b * B_b)[i][j] + beta * C
 * with the gfx950 instruction v_mfma_scale_f32_32x32x64_f8f6f4, whose E8M0
 * operands scale exactly these 32-element blocks.
 *   a_type, b_type  FP8_E4M3 / BF8_E5M2, any pair; FP6_E2M3 / BF6_E3M2, any
 *                   pair; or FP4_E2M1 x FP4_E2M1.  K % 32 == 0.
 *   A, B            as in mmac_gemm_dense; for FP4 and FP6 the row pitches
 *                   lda, ldb count elements: even for FP4 (the 16-byte pitch
 *                   rule applies to lda / 2 bytes), a multiple of 4 for FP6
 *                   (rows of 3 lda / 4 bytes, which must be a multiple of 16,
 *                   so lda % 64 == 0) -- MMAC_ERR_MISALIGNED otherwise.
 *   SA              scale words of A: ceil(K/128) x ldsa 32-bit words,
 *                   SA[t*ldsa + i] holds the exponents of blocks 4t .. 4t+3
 *                   of row i in its bytes 0 .. 3 (byte q: block 4t + q,
 *                   elements 32(4t+q) .. 32(4t+q)+31 along K).  ldsa >= M,
 *                   ldsa % 4 == 0, SA 16-byte aligned.  Bytes of blocks at or
 *                   past K/32 are ignored.
 *   SB              the same for the N columns of B (ldsb >= N).
 *   e = 255 (NaN in E8M0) in a block that is used gives unspecified results.
 *   C, D, ep, stream and the error rules as in mmac_gemm_dense_ep.  Outputs
 *   with M <= 32 rows use the tiled kernel (there is no skinny path here).
 */
mmac_status_t mmac_gemm_dense_mx(mmac_dtype_t a_type, mmac_dtype_t b_type,
                                 int64_t M, int64_t N, int64_t K, double alpha,
                                 const void *A, int64_t lda, const uint32_t *SA, int64_t ldsa,
                                 const void *B, int64_t ldb, const uint32_t *SB, int64_t ldsb,
                                 double beta, const void *C, int64_t ldc,
                                 void *D, int64_t ldd, const mmac_epilogue_t *ep, void *stream);

/*
 * Dense GEMM with other operand layouts.  trans_a = 1: A is stored
 * M-contiguous (column-major M x K: A[i + k*lda], lda >= M); trans_b = 1: B
 * is stored N-contiguous (row-major K x N: B[k*ldb + j], ldb >= N).
 * trans_a = trans_b = 0 is mmac_gemm_dense_ep.  The kernels copy such an
 * operand into LDS as K rows and read its fragments with the gfx950
 * transposing LDS reads (ds_read_b64_tr_b16 for 16-bit elements,
 * ds_read_b64_tr_b8 for 8-bit ones).
 *   (a_type, b_type) as in mmac_gemm_dense (MMAC_ERR_UNSUPPORTED
 *   otherwise); a transposed operand's K rows must span less than 2 GiB
 *   (K * ld * element size bytes; MMAC_ERR_UNSUPPORTED).  The 16-byte
 *   alignment and pitch rules, C, D, ep, stream and errors as in
 *   mmac_gemm_dense_ep.  Outputs with M <= 32 rows use the tiled kernel.
 *   Flags other than 0 / 1: MMAC_ERR_INVALID_ARG.
 */
mmac_status_t mmac_gemm_dense_layout(mmac_dtype_t a_type, mmac_dtype_t b_type, int trans_a, int trans_b,
                                     int64_t M, int64_t N, int64_t K, double alpha,
                                     const void *A, int64_t lda, const void *B, int64_t ldb,
                                     double beta, const void *C, int64_t ldc,
                                     void *D, int64_t ldd, const mmac_epilogue_t *ep, void *stream);

/*
 * Workspace bytes the _ws calls use for an M x N x K product with A of type
 * a_type (sparse != 0: mmac_gemm_sparse24_ws), under the current environment;
 * 0 when they would not split.  Host-only, no GPU work.
 */
int64_t mmac_gemm_workspace_bytes(mmac_dtype_t a_type, int64_t M, int64_t N, int64_t K, int sparse);

/* Static, human-readable name of a status code (never NULL). */
const char *mmac_status_string(mmac_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* MMAC_H */
