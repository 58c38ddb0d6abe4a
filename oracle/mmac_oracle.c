/*
 * mmac oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU implementation of what the GPU library
 * computes:
 *   - dense   D = alpha * A*B + beta * C       (fp64 or int64 accumulation)
 *   - 4:2 compression of a structured-sparse A into non-zeros + index nibbles
 *   - magnitude pruning of a dense A to 4:2 followed by that compression
 *   - the output epilogue variants: per-column bias, ReLU, rounding to
 *     bfloat16 / binary16 with saturation
 *   - sparse  D = alpha * A*B + beta * C with A given in compressed form
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  It shares no source, header, table or helper with the
 * HIP library: every decoder and loop below is written out here.
 *
 * Sources (ROCm handbook pages):
 *   "CDNA dense MFMA builtins", section "Naming convention": one instruction
 *     adds the contribution of a K-wide panel of A (M x K) and B (K x N) to an
 *     M x N output tile; the caller loops over K to form the full product.
 *     The oracle is that full product written out as a triple loop.
 *   "CDNA3 sparse MFMA builtins", section "Structured sparsity (4:2 pattern)":
 *     every contiguous group of four along K holds exactly two non-zeros; the
 *     compressed operand stores only those, in order, half the K length, and a
 *     per-group index names their two positions.  Section "FP8 16x16 sparse
 *     kernel": the positions {0,2} give the index value 0x8 per group (0x88 for
 *     two groups, 0x8888 for four), which fixes the nibble encoding
 *     p0 | (p1 << 2) with p0 < p1.
 *   The element formats are named on the pages (FP16, BF16, INT8, FP8 E4M3,
 *   BF8 E5M2; OCP encoding after gfx942, "CDNA3 sparse MFMA builtins", note in
 *   "FP8 16x16 sparse kernel"); their bit layouts come from IEEE 754 binary16,
 *   the bfloat16 definition (upper half of binary32) and the OCP 8-bit floating
 *   point specification.
 *
 * Layout conventions (shared with the library's public header by contract,
 * not by code): A row-major M x K (A[i*lda + k]); B column-major K x N
 * (B[j*ldb + k]); C and D row-major M x N; compressed A row-major M x K/2;
 * index row-major M x ceil(K/32) 32-bit words, group g of a row at bits
 * 4*(g mod 8) of word g/8.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F16 = 1, OR_BF16 = 2, OR_I8 = 3, OR_E4M3 = 4, OR_E5M2 = 5, OR_FP4 = 6, OR_FP6_E2M3 = 7, OR_BF6_E3M2 = 8 };

static int elem_bytes(int t) { return (t == OR_F16 || t == OR_BF16) ? 2 : 1; }
static int is_float_type(int t) {
    return t == OR_F16 || t == OR_BF16 || t == OR_E4M3 || t == OR_E5M2 || t == OR_FP4 || t == OR_FP6_E2M3 ||
           t == OR_BF6_E3M2;
}
static int is_fp6(int t) { return t == OR_FP6_E2M3 || t == OR_BF6_E3M2; }

/* Element `off` (counted in elements) of an array of type t.  FP4 packs two
 * elements per byte, element 2m in bits 0-3 and element 2m+1 in bits 4-7.
 * FP6 packs four elements in three bytes: element n occupies bits 6n .. 6n+5
 * of the array read as one little-endian bit string (bit b is bit b mod 8 of
 * byte b / 8). */
static uint32_t load_bits(int t, const void *base, int64_t off) {
    if (t == OR_FP4) return (((const uint8_t *)base)[off >> 1] >> (4 * (off & 1))) & 15u;
    if (is_fp6(t)) {
        const uint8_t *b = (const uint8_t *)base;
        const int64_t bit = 6 * off;
        uint32_t v = 0;
        for (int q = 0; q < 6; ++q) v |= (uint32_t)((b[(bit + q) >> 3] >> ((bit + q) & 7)) & 1u) << q;
        return v;
    }
    if (elem_bytes(t) == 2) return ((const uint16_t *)base)[off];
    return ((const uint8_t *)base)[off];
}

/* value = (-1)^s * 1.m * 2^(e - bias) for normals, (-1)^s * 0.m * 2^(1 - bias) for e == 0 */
static double from_fields(unsigned s, unsigned e, unsigned m, int mbits, int bias) {
    double mag;
    if (e == 0)
        mag = ldexp((double)m, 1 - bias - mbits);
    else
        mag = ldexp((double)((1u << mbits) | m), (int)e - bias - mbits);
    return s ? -mag : mag;
}

/* Decode one element of type t from its raw bits. */
double oracle_decode_one(int t, uint32_t bits) {
    unsigned s, e, m;
    switch (t) {
    case OR_F16: /* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa */
        s = (bits >> 15) & 1u; e = (bits >> 10) & 31u; m = bits & 1023u;
        if (e == 31u) return m ? NAN : (s ? -INFINITY : INFINITY);
        return from_fields(s, e, m, 10, 15);
    case OR_BF16: /* upper half of binary32: 1 sign, 8 exponent (bias 127), 7 mantissa */
        s = (bits >> 15) & 1u; e = (bits >> 7) & 255u; m = bits & 127u;
        if (e == 255u) return m ? NAN : (s ? -INFINITY : INFINITY);
        return from_fields(s, e, m, 7, 127);
    case OR_E4M3: /* OCP E4M3: bias 7, no infinities, S.1111.111 is NaN, max 448 */
        s = (bits >> 7) & 1u; e = (bits >> 3) & 15u; m = bits & 7u;
        if (e == 15u && m == 7u) return NAN;
        return from_fields(s, e, m, 3, 7);
    case OR_E5M2: /* OCP E5M2: bias 15, S.11111.00 is infinity, S.11111.xx (xx != 0) NaN */
        s = (bits >> 7) & 1u; e = (bits >> 2) & 31u; m = bits & 3u;
        if (e == 31u) return m ? NAN : (s ? -INFINITY : INFINITY);
        return from_fields(s, e, m, 2, 15);
    case OR_FP4: /* OCP FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa; no infinities or NaN, max 6 */
        s = (bits >> 3) & 1u; e = (bits >> 1) & 3u; m = bits & 1u;
        return from_fields(s, e, m, 1, 1);
    case OR_FP6_E2M3: /* OCP FP6 E2M3: 1 sign, 2 exponent (bias 1), 3 mantissa; no infinities or NaN, max 7.5 */
        s = (bits >> 5) & 1u; e = (bits >> 3) & 3u; m = bits & 7u;
        return from_fields(s, e, m, 3, 1);
    case OR_BF6_E3M2: /* OCP FP6 E3M2: 1 sign, 3 exponent (bias 3), 2 mantissa; no infinities or NaN, max 28 */
        s = (bits >> 5) & 1u; e = (bits >> 2) & 7u; m = bits & 3u;
        return from_fields(s, e, m, 2, 3);
    case OR_I8: /* two's complement */
        return (double)(int8_t)(uint8_t)bits;
    default:
        return NAN;
    }
}

/* Decode n elements of type t into doubles.  Returns 0, or -1 on a bad type. */
int oracle_decode(int t, int64_t n, const void *src, double *dst) {
    if (t < OR_F16 || t > OR_BF6_E3M2) return -1;
    for (int64_t q = 0; q < n; ++q) dst[q] = oracle_decode_one(t, load_bits(t, src, q));
    return 0;
}

static int bad_float_pair(int ta, int tb) {
    if (ta == OR_F16 || ta == OR_BF16 || ta == OR_FP4) return tb != ta;
    if (ta == OR_E4M3 || ta == OR_E5M2) return !(tb == OR_E4M3 || tb == OR_E5M2);
    if (is_fp6(ta)) return !is_fp6(tb);
    return 1;
}

/* Decode the whole of B (column-major, K x N) into Bd[j*K + k]. */
static double *decode_b(int tb, int64_t N, int64_t K, const void *B, int64_t ldb) {
    double *Bd = (double *)malloc((size_t)(N * K > 0 ? N * K : 1) * sizeof(double));
    if (!Bd) return NULL;
    for (int64_t j = 0; j < N; ++j)
        for (int64_t k = 0; k < K; ++k) Bd[j * K + k] = oracle_decode_one(tb, load_bits(tb, B, j * ldb + k));
    return Bd;
}

/*
 * Dense floating GEMM, rows [r0, r1) of the output:
 *   D[i-r0][j] = alpha * sum_{k ascending} A[i,k]*B[k,j] + beta * C[i,j]
 * accumulated in fp64.  beta == 0 means C is not read (C may be NULL).
 * S (optional, same shape as D) receives sum_k |A[i,k]*B[k,j]|, the scale the
 * tests use for their normwise error.
 */
int oracle_gemm_dense_f64(int ta, int tb, int64_t M, int64_t N, int64_t K, double alpha,
                          const void *A, int64_t lda, const void *B, int64_t ldb,
                          double beta, const float *C, int64_t ldc,
                          int64_t r0, int64_t r1, double *D, int64_t ldd, double *S, int64_t lds) {
    if (bad_float_pair(ta, tb) || M < 0 || N < 0 || K < 0 || r0 < 0 || r1 > M || r0 > r1) return -1;
    if (beta != 0.0 && !C) return -1;
    double *Bd = decode_b(tb, N, K, B, ldb);
    if (!Bd) return -2;
    int rc = 0;
#pragma omp parallel
    {
        double *Ad = (double *)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
        if (!Ad) {
#pragma omp atomic write
            rc = -2;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = r0; i < r1; ++i) {
                for (int64_t k = 0; k < K; ++k) Ad[k] = oracle_decode_one(ta, load_bits(ta, A, i * lda + k));
                for (int64_t j = 0; j < N; ++j) {
                    const double *bj = Bd + j * K;
                    double acc = 0.0, sabs = 0.0;
                    for (int64_t k = 0; k < K; ++k) {
                        double p = Ad[k] * bj[k];
                        acc += p;
                        sabs += fabs(p);
                    }
                    double d = alpha * acc;
                    if (beta != 0.0) d += beta * (double)C[i * ldc + j];
                    D[(i - r0) * ldd + j] = d;
                    if (S) S[(i - r0) * lds + j] = sabs;
                }
            }
            free(Ad);
        }
    }
    free(Bd);
    return rc;
}

/*
 * Block-scaled ("microscaling", MX) GEMM -- beyond the pages, from the OCP
 * Microscaling Formats specification: along K every block of 32 consecutive
 * elements of a row of A (and of a column of B) shares one E8M0 scale, an
 * unsigned 8-bit exponent with value 2^(e - 127) (e = 255 is NaN).  The
 * product is
 *   D[i][j] = alpha * sum_b 2^(SA[i][b] - 127) * 2^(SB[j][b] - 127)
 *                         * sum_{k in block b} a[i][k] * b[k][j]  +  beta * C[i][j]
 * summed exactly in fp64 (every term is a power-of-two multiple of an exact
 * product of two elements).  The elements are fp8 (E4M3 / E5M2, any pair),
 * FP6 (E2M3 / E3M2, any pair) or FP4 (E2M1 with E2M1), the element formats
 * of that specification.  SA is M x K/32 bytes (row pitch ldsa), SB is N x K/32 bytes
 * (ldsb), both row-major; K must be a multiple of 32.  S receives
 * sum |scaled product|, the error scale.  Rows [r0, r1) as in the dense oracle.
 */
static double e8m0(uint8_t e) { return e == 255 ? NAN : ldexp(1.0, (int)e - 127); }

int oracle_gemm_mx_f64(int ta, int tb, int64_t M, int64_t N, int64_t K, double alpha,
                       const void *A, int64_t lda, const uint8_t *SA, int64_t ldsa,
                       const void *B, int64_t ldb, const uint8_t *SB, int64_t ldsb,
                       double beta, const float *C, int64_t ldc,
                       int64_t r0, int64_t r1, double *D, int64_t ldd, double *S, int64_t lds) {
    if (bad_float_pair(ta, tb) || M < 0 || N < 0 || K < 0 || (K % 32) != 0 || r0 < 0 || r1 > M || r0 > r1) return -1;
    if (beta != 0.0 && !C) return -1;
    double *Bd = decode_b(tb, N, K, B, ldb);
    if (!Bd) return -2;
    const int64_t nb = K / 32;
    int rc = 0;
#pragma omp parallel
    {
        double *Ad = (double *)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
        if (!Ad) {
#pragma omp atomic write
            rc = -2;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = r0; i < r1; ++i) {
                for (int64_t k = 0; k < K; ++k) Ad[k] = oracle_decode_one(ta, load_bits(ta, A, i * lda + k));
                for (int64_t j = 0; j < N; ++j) {
                    const double *bj = Bd + j * K;
                    double acc = 0.0, sabs = 0.0;
                    for (int64_t b = 0; b < nb; ++b) {
                        const double scale = e8m0(SA[i * ldsa + b]) * e8m0(SB[j * ldsb + b]);
                        for (int64_t k = 32 * b; k < 32 * b + 32; ++k) {
                            double p = scale * (Ad[k] * bj[k]);
                            acc += p;
                            sabs += fabs(p);
                        }
                    }
                    double d = alpha * acc;
                    if (beta != 0.0) d += beta * (double)C[i * ldc + j];
                    D[(i - r0) * ldd + j] = d;
                    if (S) S[(i - r0) * lds + j] = sabs;
                }
            }
            free(Ad);
        }
    }
    free(Bd);
    return rc;
}

/* The block-scaled GEMM at n individual output positions. */
int oracle_gemm_mx_f64_entries(int ta, int tb, int64_t M, int64_t N, int64_t K, double alpha,
                               const void *A, int64_t lda, const uint8_t *SA, int64_t ldsa,
                               const void *B, int64_t ldb, const uint8_t *SB, int64_t ldsb,
                               double beta, const float *C, int64_t ldc,
                               int64_t n, const int64_t *ii, const int64_t *jj, double *out, double *S) {
    if (bad_float_pair(ta, tb) || M < 0 || N < 0 || K < 0 || (K % 32) != 0) return -1;
    if (beta != 0.0 && !C) return -1;
    for (int64_t q = 0; q < n; ++q)
        if (ii[q] < 0 || ii[q] >= M || jj[q] < 0 || jj[q] >= N) return -1;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t q = 0; q < n; ++q) {
        const int64_t i = ii[q], j = jj[q];
        double acc = 0.0, sabs = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double scale = e8m0(SA[i * ldsa + k / 32]) * e8m0(SB[j * ldsb + k / 32]);
            double p = scale * (oracle_decode_one(ta, load_bits(ta, A, i * lda + k)) *
                                oracle_decode_one(tb, load_bits(tb, B, j * ldb + k)));
            acc += p;
            sabs += fabs(p);
        }
        double d = alpha * acc;
        if (beta != 0.0) d += beta * (double)C[i * ldc + j];
        out[q] = d;
        if (S) S[q] = sabs;
    }
    return 0;
}

/* Dense floating GEMM at n individual output positions (ii[q], jj[q]). */
int oracle_gemm_dense_f64_entries(int ta, int tb, int64_t M, int64_t N, int64_t K, double alpha,
                                  const void *A, int64_t lda, const void *B, int64_t ldb,
                                  double beta, const float *C, int64_t ldc,
                                  int64_t n, const int64_t *ii, const int64_t *jj, double *out, double *S) {
    if (bad_float_pair(ta, tb) || M < 0 || N < 0 || K < 0) return -1;
    if (beta != 0.0 && !C) return -1;
    for (int64_t q = 0; q < n; ++q)
        if (ii[q] < 0 || ii[q] >= M || jj[q] < 0 || jj[q] >= N) return -1;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t q = 0; q < n; ++q) {
        int64_t i = ii[q], j = jj[q];
        double acc = 0.0, sabs = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = oracle_decode_one(ta, load_bits(ta, A, i * lda + k)) *
                       oracle_decode_one(tb, load_bits(tb, B, j * ldb + k));
            acc += p;
            sabs += fabs(p);
        }
        double d = alpha * acc;
        if (beta != 0.0) d += beta * (double)C[i * ldc + j];
        out[q] = d;
        if (S) S[q] = sabs;
    }
    return 0;
}

/*
 * Exact value v reduced to int32 by two's complement wrap (mod 2^32).
 * *oor is set to 1 when v itself lies outside int32.
 */
static int32_t wrap_i32(__int128 v, int *oor) {
    if (v < (__int128)INT32_MIN || v > (__int128)INT32_MAX) *oor = 1;
    uint32_t lo = (uint32_t)((unsigned __int128)v & 0xffffffffu);
    return (int32_t)lo;
}

/*
 * Dense int8 GEMM, rows [r0, r1):  D = alpha * sum_k A*B + beta * C, computed
 * exactly (int64 sum, 128-bit epilogue), then wrapped to int32.  beta == 0 means
 * C is not read.  *out_of_range (optional) is set to 1 if any exact value left
 * int32 before the wrap.
 */
int oracle_gemm_dense_i8(int64_t M, int64_t N, int64_t K, int64_t alpha,
                         const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb,
                         int64_t beta, const int32_t *C, int64_t ldc,
                         int64_t r0, int64_t r1, int32_t *D, int64_t ldd, int *out_of_range) {
    if (M < 0 || N < 0 || K < 0 || r0 < 0 || r1 > M || r0 > r1) return -1;
    if (beta != 0 && !C) return -1;
    int oor = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : oor)
    for (int64_t i = r0; i < r1; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k) acc += (int64_t)A[i * lda + k] * (int64_t)B[j * ldb + k];
            __int128 v = (__int128)alpha * acc;
            if (beta != 0) v += (__int128)beta * C[i * ldc + j];
            D[(i - r0) * ldd + j] = wrap_i32(v, &oor);
        }
    }
    if (out_of_range) *out_of_range = oor;
    return 0;
}

/* Is this element a zero?  Floating types: both signed zeros; int8: only 0. */
static int elem_is_zero(int t, uint32_t bits) {
    switch (t) {
    case OR_F16:
    case OR_BF16: return (bits & 0x7fffu) == 0;
    case OR_E4M3:
    case OR_E5M2: return (bits & 0x7fu) == 0;
    default: return bits == 0;
    }
}

static void store_bits(int t, void *base, int64_t off, uint32_t bits) {
    if (elem_bytes(t) == 2) ((uint16_t *)base)[off] = (uint16_t)bits;
    else ((uint8_t *)base)[off] = (uint8_t)bits;
}

/*
 * Reference 4:2 compressor ("CDNA3 sparse MFMA builtins", "Structured sparsity
 * (4:2 pattern)"): walk each row of A along K in groups of four, find the
 * positions of the non-zeros, and store those two values one after the other.
 *
 *   - non-zero: any element that is not +0/-0 (floating) or 0 (int8); a NaN
 *     counts as non-zero;
 *   - more than two non-zeros: the group violates the pattern; keep the two
 *     lowest positions and count the group in *bad_groups;
 *   - fewer than two: pad with the lowest unused positions (their stored
 *     value is the zero found there, copied bit for bit), so p0 < p1 always;
 *   - nibble = p0 | (p1 << 2); group g of a row sits at bits 4*(g mod 8) of
 *     index word g/8; bits of groups past K/4 are zero.
 * K must be a multiple of 4.  Returns 0, or -1 on bad arguments.
 */
int oracle_compress24(int t, int64_t M, int64_t K, const void *A, int64_t lda,
                      void *Ac, int64_t ldac, uint32_t *idx, int64_t ldidx, int64_t *bad_groups) {
    if (t < OR_F16 || t > OR_E5M2 || M < 0 || K < 0 || (K % 4) != 0) return -1;
    const int64_t G = K / 4, words = (K + 31) / 32;
    int64_t bad = 0;
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t w = 0; w < words; ++w) idx[i * ldidx + w] = 0u;
        for (int64_t g = 0; g < G; ++g) {
            int pos[4], np = 0;
            for (int p = 0; p < 4; ++p)
                if (!elem_is_zero(t, load_bits(t, A, i * lda + 4 * g + p))) pos[np++] = p;
            if (np > 2) { ++bad; np = 2; }
            /* pad with the lowest positions not yet taken */
            for (int p = 0; p < 4 && np < 2; ++p) {
                int taken = 0;
                for (int q = 0; q < np; ++q) taken |= (pos[q] == p);
                if (!taken) pos[np++] = p;
            }
            if (pos[0] > pos[1]) { int tmp = pos[0]; pos[0] = pos[1]; pos[1] = tmp; }
            store_bits(t, Ac, i * ldac + 2 * g, load_bits(t, A, i * lda + 4 * g + pos[0]));
            store_bits(t, Ac, i * ldac + 2 * g + 1, load_bits(t, A, i * lda + 4 * g + pos[1]));
            uint32_t nib = (uint32_t)pos[0] | ((uint32_t)pos[1] << 2);
            idx[i * ldidx + g / 8] |= nib << (4 * (g % 8));
        }
    }
    if (bad_groups) *bad_groups = bad;
    return 0;
}

/*
 * Output epilogue variants (beyond the pages, which accumulate in fp32/int32
 * and return that): from the exact value y = alpha*A*B + beta*C of the plain
 * GEMM, add a per-column bias, apply an activation, then round to the output
 * format.
 *   activation 0: none; 1: ReLU, max(y, 0) (a NaN stays NaN);
 *   output 1: bfloat16, 2: IEEE binary16 (3, 4: OCP fp8, below); rounding to
 *   nearest, ties to even (from the exact value), saturating: a finite value
 *   beyond the largest finite magnitude becomes that magnitude with its
 *   sign; infinities stay infinities, a NaN becomes the format's quiet NaN
 *   with the same sign.
 */
static uint32_t round_to_format(double y, int mant_bits, int exp_bits) {
    const int bias = (1 << (exp_bits - 1)) - 1, emax = bias, emin = 1 - bias;
    const uint32_t sign = signbit(y) ? 1u : 0u;
    const uint32_t exp_all = (1u << exp_bits) - 1u, total = 1u + (uint32_t)exp_bits + (uint32_t)mant_bits;
    const uint32_t sbit = sign << (total - 1);
    if (isnan(y)) return sbit | (exp_all << mant_bits) | (1u << (mant_bits - 1));
    if (isinf(y)) return sbit | (exp_all << mant_bits);
    double a = fabs(y);
    const double max_finite = ldexp(2.0 - ldexp(1.0, -mant_bits), emax);
    /* quantum of the binade holding a (subnormal quantum below 2^emin) */
    int e = (a > 0.0) ? ilogb(a) : emin;
    if (e < emin) e = emin;
    const double q = ldexp(1.0, e - mant_bits);
    double n = a / q;                         /* exact: a is a double, q a power of two */
    double r = floor(n);
    const double frac = n - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    double v = r * q;                         /* rounded magnitude (may reach the next binade) */
    if (v > max_finite) v = max_finite;       /* saturate */
    if (v == 0.0) return sbit;
    int ev = ilogb(v);
    uint32_t field, mant;
    if (ev < emin) {                          /* subnormal */
        field = 0u;
        mant = (uint32_t)(v / ldexp(1.0, emin - mant_bits));
    } else {
        field = (uint32_t)(ev + bias);
        mant = (uint32_t)((v / ldexp(1.0, ev) - 1.0) * ldexp(1.0, mant_bits));
    }
    return sbit | (field << mant_bits) | mant;
}

/*
 * Rounding to the OCP 8-bit floats (the fp8 encodings gfx950 uses: "CDNA3
 * sparse MFMA builtins", note under the FP8 sparse kernel; OCP 8-bit floating
 * point formats):
 *   E4M3 (out_type 3): exponent bias 7, 3 fraction bits, subnormal quantum
 *     2^-9, largest finite 448 = 1.75 * 2^8 (code 0x7E: the all-ones exponent
 *     still holds normal numbers except fraction 111, which is NaN), no
 *     infinities;
 *   E5M2 (out_type 4): bias 15, 2 fraction bits, subnormal quantum 2^-16,
 *     largest finite 57344 = 1.75 * 2^15, infinities 0x7C, NaNs above.
 * To nearest, ties to even, from the exact value, saturating as above; an
 * infinity stays infinite in E5M2 and becomes the largest finite value in
 * E4M3 (which has none); NaN becomes 0x7F (E4M3) / 0x7E (E5M2), sign kept.
 */
static uint32_t round_to_fp8(double y, int e4m3) {
    const int mant_bits = e4m3 ? 3 : 2, bias = e4m3 ? 7 : 15;
    const double max_finite = e4m3 ? 448.0 : 57344.0;
    const uint32_t sbit = signbit(y) ? 0x80u : 0u;
    if (isnan(y)) return sbit | (e4m3 ? 0x7Fu : 0x7Eu);
    if (isinf(y)) return sbit | (e4m3 ? 0x7Eu : 0x7Cu);
    const double a = fabs(y);
    const int emin = 1 - bias;
    int e = (a > 0.0) ? ilogb(a) : emin;
    if (e < emin) e = emin;
    const double q = ldexp(1.0, e - mant_bits);       /* quantum of a's binade */
    const double n = a / q;                           /* exact */
    double r = floor(n);
    const double frac = n - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    double v = r * q;
    if (v > max_finite) v = max_finite;               /* saturate */
    if (v == 0.0) return sbit;
    const int ev = ilogb(v);
    if (ev < emin) return sbit | (uint32_t)(v / ldexp(1.0, emin - mant_bits));        /* subnormal */
    const uint32_t mant = (uint32_t)((v / ldexp(1.0, ev) - 1.0) * ldexp(1.0, mant_bits));
    return sbit | ((uint32_t)(ev + bias) << mant_bits) | mant;
}

/* One output element of the given type: bits (1 bfloat16, 2 binary16, 3 E4M3, 4 E5M2). */
static uint32_t round_out(int out_type, double y) {
    switch (out_type) {
    case 1: return round_to_format(y, 7, 8);
    case 2: return round_to_format(y, 10, 5);
    case 3: return round_to_fp8(y, 1);
    default: return round_to_fp8(y, 0);
    }
}

int oracle_epilogue(int64_t M, int64_t N, const double *Y, int64_t ldy, const float *bias, int act, int out_type,
                    void *out, int64_t ldo, double *Yout) {
    if (M < 0 || N < 0 || act < 0 || act > 1 || out_type < 0 || out_type > 4) return -1;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            double y = Y[i * ldy + j];
            if (bias) y += (double)bias[j];
            if (act == 1 && y < 0.0) y = 0.0;
            if (Yout) Yout[i * ldo + j] = y;
            if (out_type == 1 || out_type == 2) ((uint16_t *)out)[i * ldo + j] = (uint16_t)round_out(out_type, y);
            else if (out_type >= 3) ((uint8_t *)out)[i * ldo + j] = (uint8_t)round_out(out_type, y);
            else ((float *)out)[i * ldo + j] = (float)y;
        }
    return 0;
}

/* Round n doubles to bfloat16 (out_type 1), binary16 (2), E4M3 (3) or E5M2 (4) bits, as above
 * (for the pins; 8-bit results are returned in the low byte of each 16-bit word). */
int oracle_round(int out_type, int64_t n, const double *x, uint16_t *bits) {
    if (out_type < 1 || out_type > 4) return -1;
    for (int64_t q = 0; q < n; ++q) bits[q] = (uint16_t)round_out(out_type, x[q]);
    return 0;
}

/*
 * Magnitude pruning to the 4:2 pattern, then compression.  The pages give the
 * pattern and the compressed form ("CDNA3 sparse MFMA builtins", "Structured
 * sparsity (4:2 pattern)") but not how a dense A is brought to it; this
 * follows the usual magnitude rule:
 *   - in every group of four along K keep the two elements of largest |a|
 *     (decoded value; int8 -128 has magnitude 128);
 *   - a NaN is larger than every number, infinities included; all NaNs tie;
 *   - ties go to the lower position;
 *   - the two kept elements are then stored exactly as the compressor above
 *     stores them (ascending positions, bits copied, nibble p0 | (p1 << 2)).
 * *bad_groups counts the groups that held more than two non-zeros (the ones
 * pruning changed), with the compressor's notion of non-zero.
 */
static int mag_greater(double x, double y) {   /* |x| > |y| with NaN above everything */
    int nx = isnan(x), ny = isnan(y);
    if (nx || ny) return nx && !ny;
    return fabs(x) > fabs(y);
}

int oracle_prune_compress24(int t, int64_t M, int64_t K, const void *A, int64_t lda,
                            void *Ac, int64_t ldac, uint32_t *idx, int64_t ldidx, int64_t *bad_groups) {
    if (t < OR_F16 || t > OR_E5M2 || M < 0 || K < 0 || (K % 4) != 0) return -1;
    const int64_t G = K / 4, words = (K + 31) / 32;
    int64_t bad = 0;
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t w = 0; w < words; ++w) idx[i * ldidx + w] = 0u;
        for (int64_t g = 0; g < G; ++g) {
            double v[4];
            int order[4], nz = 0;
            for (int p = 0; p < 4; ++p) {
                uint32_t b = load_bits(t, A, i * lda + 4 * g + p);
                v[p] = oracle_decode_one(t, b);
                nz += !elem_is_zero(t, b);
                order[p] = p;
            }
            if (nz > 2) ++bad;
            /* stable insertion sort of the positions by decreasing magnitude */
            for (int a = 1; a < 4; ++a)
                for (int b = a; b > 0 && mag_greater(v[order[b]], v[order[b - 1]]); --b) {
                    int tmp = order[b]; order[b] = order[b - 1]; order[b - 1] = tmp;
                }
            int p0 = order[0], p1 = order[1];
            if (p0 > p1) { int tmp = p0; p0 = p1; p1 = tmp; }
            store_bits(t, Ac, i * ldac + 2 * g, load_bits(t, A, i * lda + 4 * g + p0));
            store_bits(t, Ac, i * ldac + 2 * g + 1, load_bits(t, A, i * lda + 4 * g + p1));
            idx[i * ldidx + g / 8] |= ((uint32_t)p0 | ((uint32_t)p1 << 2)) << (4 * (g % 8));
        }
    }
    if (bad_groups) *bad_groups = bad;
    return 0;
}

/* Read nibble g of row i; return 0 and (p0, p1) if it is a valid pair p0 < p1. */
static int read_nibble(const uint32_t *idx, int64_t ldidx, int64_t i, int64_t g, int *p0, int *p1) {
    uint32_t nib = (idx[i * ldidx + g / 8] >> (4 * (g % 8))) & 0xfu;
    *p0 = (int)(nib & 3u);
    *p1 = (int)((nib >> 2) & 3u);
    return (*p0 < *p1) ? 0 : -1;
}

/*
 * Inverse of the compressor: rebuild the dense M x K row-major A from the
 * compressed values and index.  Positions not named by a nibble get +0 (all
 * bits clear).  Returns -1 if any nibble is not a valid pair p0 < p1.
 */
int oracle_decompress24(int t, int64_t M, int64_t K, const void *Ac, int64_t ldac,
                        const uint32_t *idx, int64_t ldidx, void *A, int64_t lda) {
    if (t < OR_F16 || t > OR_E5M2 || M < 0 || K < 0 || (K % 4) != 0) return -1;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t g = 0; g < K / 4; ++g) {
            int p0, p1;
            if (read_nibble(idx, ldidx, i, g, &p0, &p1)) return -1;
            for (int p = 0; p < 4; ++p) store_bits(t, A, i * lda + 4 * g + p, 0u);
            store_bits(t, A, i * lda + 4 * g + p0, load_bits(t, Ac, i * ldac + 2 * g));
            store_bits(t, A, i * lda + 4 * g + p1, load_bits(t, Ac, i * ldac + 2 * g + 1));
        }
    return 0;
}

/*
 * Sparse floating GEMM from the compressed form, rows [r0, r1):
 *   acc = sum_g ( Ac[i,2g]*B[4g+p0, j] + Ac[i,2g+1]*B[4g+p1, j] ),  g ascending,
 * i.e. the dense sum restricted to the two stored positions of each group, in
 * ascending K order; the epilogue is the dense one.
 */
int oracle_gemm_sparse24_f64(int ta, int tb, int64_t M, int64_t N, int64_t K, double alpha,
                             const void *Ac, int64_t ldac, const uint32_t *idx, int64_t ldidx,
                             const void *B, int64_t ldb, double beta, const float *C, int64_t ldc,
                             int64_t r0, int64_t r1, double *D, int64_t ldd, double *S, int64_t lds) {
    if (bad_float_pair(ta, tb) || M < 0 || N < 0 || K < 0 || (K % 4) != 0 || r0 < 0 || r1 > M || r0 > r1)
        return -1;
    if (beta != 0.0 && !C) return -1;
    const int64_t G = K / 4;
    for (int64_t i = r0; i < r1; ++i)
        for (int64_t g = 0; g < G; ++g) {
            int p0, p1;
            if (read_nibble(idx, ldidx, i, g, &p0, &p1)) return -1;
        }
    double *Bd = decode_b(tb, N, K, B, ldb);
    if (!Bd) return -2;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = r0; i < r1; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            const double *bj = Bd + j * K;
            double acc = 0.0, sabs = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                int p0, p1;
                read_nibble(idx, ldidx, i, g, &p0, &p1);
                double p = oracle_decode_one(ta, load_bits(ta, Ac, i * ldac + 2 * g)) * bj[4 * g + p0];
                double q = oracle_decode_one(ta, load_bits(ta, Ac, i * ldac + 2 * g + 1)) * bj[4 * g + p1];
                acc += p;
                acc += q;
                sabs += fabs(p) + fabs(q);
            }
            double d = alpha * acc;
            if (beta != 0.0) d += beta * (double)C[i * ldc + j];
            D[(i - r0) * ldd + j] = d;
            if (S) S[(i - r0) * lds + j] = sabs;
        }
    }
    free(Bd);
    return 0;
}

/* Sparse floating GEMM at n individual output positions (ii[q], jj[q]). */
int oracle_gemm_sparse24_f64_entries(int ta, int tb, int64_t M, int64_t N, int64_t K, double alpha,
                                     const void *Ac, int64_t ldac, const uint32_t *idx, int64_t ldidx,
                                     const void *B, int64_t ldb, double beta, const float *C, int64_t ldc,
                                     int64_t n, const int64_t *ii, const int64_t *jj, double *out, double *S) {
    if (bad_float_pair(ta, tb) || M < 0 || N < 0 || K < 0 || (K % 4) != 0) return -1;
    if (beta != 0.0 && !C) return -1;
    const int64_t G = K / 4;
    for (int64_t q = 0; q < n; ++q) {
        if (ii[q] < 0 || ii[q] >= M || jj[q] < 0 || jj[q] >= N) return -1;
        for (int64_t g = 0; g < G; ++g) {
            int p0, p1;
            if (read_nibble(idx, ldidx, ii[q], g, &p0, &p1)) return -1;
        }
    }
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t q = 0; q < n; ++q) {
        int64_t i = ii[q], j = jj[q];
        double acc = 0.0, sabs = 0.0;
        for (int64_t g = 0; g < G; ++g) {
            int p0, p1;
            read_nibble(idx, ldidx, i, g, &p0, &p1);
            double p = oracle_decode_one(ta, load_bits(ta, Ac, i * ldac + 2 * g)) *
                       oracle_decode_one(tb, load_bits(tb, B, j * ldb + 4 * g + p0));
            double r = oracle_decode_one(ta, load_bits(ta, Ac, i * ldac + 2 * g + 1)) *
                       oracle_decode_one(tb, load_bits(tb, B, j * ldb + 4 * g + p1));
            acc += p;
            acc += r;
            sabs += fabs(p) + fabs(r);
        }
        double d = alpha * acc;
        if (beta != 0.0) d += beta * (double)C[i * ldc + j];
        out[q] = d;
        if (S) S[q] = sabs;
    }
    return 0;
}

/* Sparse int8 GEMM from the compressed form, rows [r0, r1); exact, wrapped to int32. */
int oracle_gemm_sparse24_i8(int64_t M, int64_t N, int64_t K, int64_t alpha,
                            const int8_t *Ac, int64_t ldac, const uint32_t *idx, int64_t ldidx,
                            const int8_t *B, int64_t ldb, int64_t beta, const int32_t *C, int64_t ldc,
                            int64_t r0, int64_t r1, int32_t *D, int64_t ldd, int *out_of_range) {
    if (M < 0 || N < 0 || K < 0 || (K % 4) != 0 || r0 < 0 || r1 > M || r0 > r1) return -1;
    if (beta != 0 && !C) return -1;
    const int64_t G = K / 4;
    for (int64_t i = r0; i < r1; ++i)
        for (int64_t g = 0; g < G; ++g) {
            int p0, p1;
            if (read_nibble(idx, ldidx, i, g, &p0, &p1)) return -1;
        }
    int oor = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : oor)
    for (int64_t i = r0; i < r1; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            int64_t acc = 0;
            for (int64_t g = 0; g < G; ++g) {
                int p0, p1;
                read_nibble(idx, ldidx, i, g, &p0, &p1);
                acc += (int64_t)Ac[i * ldac + 2 * g] * (int64_t)B[j * ldb + 4 * g + p0];
                acc += (int64_t)Ac[i * ldac + 2 * g + 1] * (int64_t)B[j * ldb + 4 * g + p1];
            }
            __int128 v = (__int128)alpha * acc;
            if (beta != 0) v += (__int128)beta * C[i * ldc + j];
            D[(i - r0) * ldd + j] = wrap_i32(v, &oor);
        }
    }
    if (out_of_range) *out_of_range = oor;
    return 0;
}

/* Tell the caller whether a type code is a floating type (used by the wrapper). */
int oracle_is_float_type(int t) { return is_float_type(t); }

/* Number of threads the oracle's parallel loops use. */
int oracle_num_threads(void) { return omp_get_max_threads(); }

/* Set the thread count of later oracle calls (n >= 1); timing only, results do not depend on it. */
void oracle_set_num_threads(int n) {
    if (n >= 1) omp_set_num_threads(n);
}
