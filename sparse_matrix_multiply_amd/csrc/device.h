// Device primitives for the gfx950 GEMM kernels: fragment types, buffer
// resources, the LDS swizzle and one wrapper per matrix instruction.
//
// Fragment convention used by every kernel here.  A matrix instruction with a
// 32 x 32 output tile takes, in each of the 64 lanes, one row of A (lane mod
// 32) and one column of B (lane mod 32); the two lane halves (g = lane / 32)
// carry two different K slices of that row / column.  For a dense product the
// order in which K values sit in the lanes does not change the sum as long as
// A and B use the same order, and this library gives lane half g the g-th
// contiguous half of the instruction's K step for both.  The sparse
// instructions fix the pairing of compressed A, index and dense B (described
// above their wrappers below).  The output tile uses
// the one-block 32 x 32 accumulator layout ("CDNA dense MFMA builtins",
// "Accumulator layout", 32x32 layout; "CDNA3 sparse MFMA builtins",
// "Accumulator layout": sparse instructions use the same one-block layout).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmac {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x16 __attribute__((ext_vector_type(16)));

enum : int { DT_F16 = 1, DT_BF16 = 2, DT_I8 = 3, DT_E4M3 = 4, DT_E5M2 = 5, DT_FP4 = 6, DT_FP6 = 7, DT_BF6 = 8 };

// Word 3 of a gfx9 buffer descriptor for raw (untyped) 32-bit accesses.
constexpr int kBufferWord3 = 0x00020000;
// A byte offset that is never inside any buffer this library builds: loads
// from it return zero.
constexpr uint32_t kOutOfRange = 0x80000000u;
// Cache-policy operand of buffer loads/stores: non-temporal (the nt bit), for
// data touched once -- C read at a tile's start and D written at its end -- so
// it streams past the caches instead of evicting the A and B panels that
// other tiles still reuse.
constexpr int kNonTemporal = 2;
// Cache-policy operand for device-scope (agent-scope) accesses: the SC1 bit.
// Such a store is written through to the memory side of the L2 caches, and
// such a load is served from there, so data one XCD writes is seen by
// another without cache-wide write-back or invalidation.
constexpr int kDeviceScope = 16;

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kBufferWord3);
}

// ---- output conversions --------------------------------------------------
// Element types of C and D besides the accumulator type (float / int32).
enum : int { OUT_ACC = 0, OUT_BF16 = 1, OUT_F16 = 2, OUT_E4M3 = 3, OUT_E5M2 = 4 };

// Bytes of one C / D element of output type OT.
template <int OT> constexpr int out_esize() { return OT == OUT_ACC ? 4 : OT <= OUT_F16 ? 2 : 1; }

// fp32 -> bfloat16 bits: round to nearest, ties to even; a finite value whose
// rounding would leave the finite range gives the largest finite value of its
// sign (saturation); infinities stay infinite; NaN gives the quiet NaN 0x7fc0
// with the sign kept.  bfloat16 is the top half of an fp32, so rounding the
// low 16 bits away (with the carry into the exponent) is the whole conversion,
// subnormals included.
__device__ __forceinline__ uint32_t to_bf16_sat(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v), s = (u >> 16) & 0x8000u, a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return s | 0x7fc0u;
    if (a == 0x7f800000u) return s | 0x7f80u;
    const uint32_t h = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    return (h & 0x7fffu) == 0x7f80u ? (s | 0x7f7fu) : h;
}

// fp32 -> IEEE binary16 bits with the same rules (largest finite 65504; the
// quiet NaN is 0x7e00).  Normal results: move the exponent from bias 127 to
// bias 15 and round the 13 dropped significand bits to nearest even (a carry
// moves into the exponent, as it should).  Subnormal results (|v| < 2^-14):
// the quantum is 2^-24, so |v| * 2^24 (exact) rounded to the nearest integer,
// ties to even, is the significand field; 1024 there is the smallest normal.
__device__ __forceinline__ uint32_t to_f16_sat(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v), s = (u >> 16) & 0x8000u, a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return s | 0x7e00u;
    if (a == 0x7f800000u) return s | 0x7c00u;
    if (a >= 0x477ff000u) return s | 0x7bffu;          // |v| >= 65520 rounds past 65504
    if (a >= 0x38800000u) {                              // |v| >= 2^-14
        const uint32_t m = a - 0x38000000u;
        return s | ((m + 0xfffu + ((m >> 13) & 1u)) >> 13);
    }
    return s | (uint32_t)__builtin_rintf(__builtin_bit_cast(float, a) * 16777216.0f);
}

// fp32 -> OCP fp8 bits with the same rules.  E4M3 (bias 7, 3 fraction
// bits): largest finite 448 (0x7E), no infinities, so infinities saturate
// too, NaN 0x7F; E5M2 (bias 15, 2 fraction bits): largest finite 57344
// (0x7B), infinity 0x7C, quiet NaN 0x7E.  Any magnitude at or above the
// largest finite value rounds (or saturates) to it, so that test comes
// first; then normal results rebias the exponent and round the dropped
// significand bits to nearest even, and subnormal ones (quantum 2^-9 /
// 2^-16) scale exactly and round with rint, as for binary16.
__device__ __forceinline__ uint32_t to_e4m3_sat(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v), s = (u >> 24) & 0x80u, a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return s | 0x7fu;
    if (a >= 0x43e00000u) return s | 0x7eu;             // |v| >= 448, infinities included
    if (a >= 0x3c800000u) {                              // |v| >= 2^-6
        const uint32_t m = a - 0x3c000000u;              // exponent rebias 127 -> 7
        return s | ((m + 0x7ffffu + ((m >> 20) & 1u)) >> 20);
    }
    return s | (uint32_t)__builtin_rintf(__builtin_bit_cast(float, a) * 512.0f);
}

__device__ __forceinline__ uint32_t to_e5m2_sat(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v), s = (u >> 24) & 0x80u, a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return s | 0x7eu;
    if (a == 0x7f800000u) return s | 0x7cu;
    if (a >= 0x47600000u) return s | 0x7bu;             // |v| >= 57344
    if (a >= 0x38800000u) {                              // |v| >= 2^-14
        const uint32_t m = a - 0x38000000u;              // exponent rebias 127 -> 15
        return s | ((m + 0xfffffu + ((m >> 21) & 1u)) >> 21);
    }
    return s | (uint32_t)__builtin_rintf(__builtin_bit_cast(float, a) * 65536.0f);
}

// Stored C element (bits) -> fp32, exact for every output type.  E5M2 is the
// top byte of a binary16 with the same exponent bias.
template <int OT>
__device__ __forceinline__ float from_out_bits(uint32_t h) {
    if constexpr (OT == OUT_BF16) {
        return __builtin_bit_cast(float, h << 16);
    } else if constexpr (OT == OUT_F16) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
    } else if constexpr (OT == OUT_E5M2) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(h << 8));
    } else if constexpr (OT == OUT_E4M3) {
        const uint32_t s = (h & 0x80u) << 24, e = (h >> 3) & 15u, m = h & 7u;
        if (e == 15u && m == 7u) return __builtin_bit_cast(float, s | 0x7fc00000u);
        if (e == 0u) {
            const float x = (float)m * 0.001953125f;     // m * 2^-9, exact
            return s ? -x : x;
        }
        return __builtin_bit_cast(float, s | ((e + 120u) << 23) | (m << 20));
    } else {
        return __builtin_bit_cast(float, h);
    }
}

// The end of every floating epilogue: v = alpha * acc + beta * C already
// formed in fp32; add the column's bias (when there is one), apply ReLU (when
// asked: negative values become +0, NaN and -0 pass), and round to D's type.
template <int OT>
__device__ __forceinline__ uint32_t finish(float v, float bias, bool has_bias, bool relu) {
    if (has_bias) v += bias;
    if (relu) v = v < 0.0f ? 0.0f : v;
    if constexpr (OT == OUT_BF16) return to_bf16_sat(v);
    else if constexpr (OT == OUT_F16) return to_f16_sat(v);
    else if constexpr (OT == OUT_E4M3) return to_e4m3_sat(v);
    else if constexpr (OT == OUT_E5M2) return to_e5m2_sat(v);
    else return __builtin_bit_cast(uint32_t, v);
}

// LDS tiles are stored in 16-byte units, W units per row (row-major).  The
// LDS of gfx950 serves 16 lanes' 16-byte reads per cycle from 64 banks (256
// bytes); the fragment reads of the kernels have 16 consecutive lanes read
// the same unit c of 16 consecutive rows.  Unit c of row r is therefore stored
// at c ^ ((r / (16 / W)) mod W) of its row: the 16/W rows that share one
// 256-byte bank row keep distinct positions, and successive bank rows are
// XOR-rotated, so those 16 reads hit 16 different 16-byte bank groups.  The
// map keeps the row and is its own inverse.
template <int W>
__device__ __forceinline__ constexpr uint32_t swz(uint32_t L) {
    static_assert(W == 2 || W == 4 || W == 8, "rows of 2, 4 or 8 units");
    const uint32_t r = L / W;
    return r * W + ((L % W) ^ ((r / (16 / W)) % W));
}

// ---- matrix-instruction wrappers -----------------------------------------
// Each describes one instruction: bytes of A and B per lane, dense K per
// instruction, accumulator and output types, and mma().

template <int BYTES> struct Frag;
template <> struct Frag<16> { i32x4 v; };
template <> struct Frag<32> { i32x4 lo, hi; };
typedef int i32x6 __attribute__((ext_vector_type(6)));
// Packed FP6 operand as read from LDS: the lane half's own 16-byte unit x and
// the 16-byte unit z that its block shares with the other half's (the
// operand is put together at the instruction, so the reads need not be
// waited for before then).
template <> struct Frag<24> { i32x4 x, z; };

__device__ __forceinline__ i32x8 join(const Frag<32> &f) {
    return i32x8{f.lo[0], f.lo[1], f.lo[2], f.lo[3], f.hi[0], f.hi[1], f.hi[2], f.hi[3]};
}

// Every op's LDS k-tile rows are 128 bytes: a copy instruction then covers
// whole 128-byte lines (8 lanes per row), and the vector L1 handles half as
// many line requests per byte as with 64-byte rows; that request rate, not
// the bytes, is what limits the copies.

// Dense bf16 / fp16: v_mfma_f32_32x32x16_{bf16,f16}, 8 elements (16 B) per lane.
template <int DT> struct MmaDense16 {
    static constexpr bool kSparse = false, kScaled = false;
    static constexpr int kScaleWords = 0;
    static constexpr int kEsize = 2, kAFrag = 16, kBFrag = 16, kKStep = 16;
    static constexpr int kBK = 64;                 // dense K per LDS k-tile
    static constexpr int kARowBytes = kBK * kEsize, kBRowBytes = kBK * kEsize;
    typedef f32x16 acc_t;
    typedef float out_t;
    // 16-byte unit (within a k-tile row) of half h of the fragment of lane half g, step s
    __device__ __forceinline__ static constexpr int a_unit(int s, int g, int) { return 2 * s + g; }
    __device__ __forceinline__ static constexpr int b_unit(int s, int g, int) { return 2 * s + g; }
    __device__ __forceinline__ static acc_t mma(const Frag<16> &a, const Frag<16> &b, acc_t c, uint32_t) {
        if constexpr (DT == DT_BF16)
            return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                          __builtin_bit_cast(bf16x8, b.v), c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a.v),
                                                         __builtin_bit_cast(f16x8, b.v), c, 0, 0, 0);
    }
};

// Dense int8: v_mfma_i32_32x32x32_i8, 16 elements (16 B) per lane.
struct MmaDenseI8 {
    static constexpr bool kSparse = false, kScaled = false;
    static constexpr int kScaleWords = 0;
    static constexpr int kEsize = 1, kAFrag = 16, kBFrag = 16, kKStep = 32;
    static constexpr int kBK = 128;
    static constexpr int kARowBytes = kBK, kBRowBytes = kBK;
    typedef i32x16 acc_t;
    typedef int32_t out_t;
    __device__ __forceinline__ static constexpr int a_unit(int s, int g, int) { return 2 * s + g; }
    __device__ __forceinline__ static constexpr int b_unit(int s, int g, int) { return 2 * s + g; }
    __device__ __forceinline__ static acc_t mma(const Frag<16> &a, const Frag<16> &b, acc_t c, uint32_t) {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(a.v, b.v, c, 0, 0, 0);
    }
};

// Dense fp8 / bf8 (OCP): v_mfma_f32_32x32x64_f8f6f4 with unit scales; the
// format selectors name the A and B formats (0 = E4M3, 1 = E5M2).
template <int FA, int FB> struct MmaDenseF8 {
    static constexpr bool kSparse = false, kScaled = false;
    static constexpr int kScaleWords = 0;
    static constexpr int kEsize = 1, kAFrag = 32, kBFrag = 32, kKStep = 64;
    static constexpr int kBK = 128;
    static constexpr int kARowBytes = kBK, kBRowBytes = kBK;
    typedef f32x16 acc_t;
    typedef float out_t;
    __device__ __forceinline__ static constexpr int a_unit(int s, int g, int h) { return 4 * s + 2 * g + h; }
    __device__ __forceinline__ static constexpr int b_unit(int s, int g, int h) { return 4 * s + 2 * g + h; }
    __device__ __forceinline__ static acc_t mma(const Frag<32> &a, const Frag<32> &b, acc_t c, uint32_t) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(join(a), join(b), c, FA, FB, 0, 0, 0, 0);
    }
};

// Block-scaled (MX) fp8 / bf8: v_mfma_scale_f32_32x32x64_f8f6f4 with E8M0
// scale operands.  The instruction's own K order within its 64-K step puts
// K 16g .. 16g+15 in the first 16 bytes of lane half g's operand and
// K 32+16g .. 32+16g+15 in the second (the order the sparse B fragments
// above also show), and scales its K block 32c .. 32c+31 with byte 0 of the
// scale operand of lane half c.  So these fragments load, for lane half g of
// step s, the 16-byte units 4s + g and 4s + 2 + g: the instruction's K order is
// then the matrix's, and lane half g's scale byte is that of block 2s + g of
// the k-tile.  Established on gfx950 with one-wave probes (lane-, row- and
// column-dependent scales, byte select) and with one-block-scaled GEMMs
// through this library (each block's exponent doubled in turn, K chunks
// weighted by distinct powers of two); every MX parity test rechecks it.
// (For the unscaled dense product the unit order does not matter: A and B
// use the same one.)  Scale words come in per k-tile: kScaleWords words of
// four block exponents per row of A and per column of B.
template <int FA, int FB> struct MmaMX : MmaDenseF8<FA, FB> {
    typedef typename MmaDenseF8<FA, FB>::acc_t acc_t;
    static constexpr bool kScaled = true;
    static constexpr int kScaleWords = MmaDenseF8<FA, FB>::kBK / 128;
    __device__ __forceinline__ static constexpr int a_unit(int s, int g, int h) { return 4 * s + g + 2 * h; }
    __device__ __forceinline__ static constexpr int b_unit(int s, int g, int h) { return 4 * s + g + 2 * h; }
    __device__ __forceinline__ static acc_t mma_scaled(const Frag<32> &a, const Frag<32> &b, acc_t c, uint32_t sa,
                                                       uint32_t sb) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(join(a), join(b), c, FA, FB, 0, (int)sa, 0, (int)sb);
    }
};

// Block-scaled (MX) FP4 E2M1 x FP4: the same instruction with format 4 on
// both sides.  A lane's operand is 16 bytes, 32 elements packed two per byte
// (low nibble first); 128-byte LDS rows hold 256 elements per k-tile, so a
// k-tile is four 64-K steps and two scale words per row.  Lane half g of
// step s loads 16-byte unit 2s + g: K 64s + 32g .. 64s + 32g + 31, block
// 2s + g.  Copies count bytes: 4 bits per element.
struct MmaMX4 {
    static constexpr bool kSparse = false, kScaled = true;
    static constexpr int kEsize = 1, kElemBits = 4, kAFrag = 16, kBFrag = 16, kKStep = 64;
    static constexpr int kBK = 256;
    static constexpr int kARowBytes = kBK / 2, kBRowBytes = kBK / 2;
    static constexpr int kScaleWords = kBK / 128;
    typedef f32x16 acc_t;
    typedef float out_t;
    __device__ __forceinline__ static constexpr int a_unit(int s, int g, int) { return 2 * s + g; }
    __device__ __forceinline__ static constexpr int b_unit(int s, int g, int) { return 2 * s + g; }
    __device__ __forceinline__ static acc_t mma_scaled(const Frag<16> &a, const Frag<16> &b, acc_t c, uint32_t sa,
                                                       uint32_t sb) {
        const i32x8 A = {a.v[0], a.v[1], a.v[2], a.v[3], 0, 0, 0, 0};
        const i32x8 B = {b.v[0], b.v[1], b.v[2], b.v[3], 0, 0, 0, 0};
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, c, 4, 4, 0, (int)sa, 0, (int)sb);
    }
};

// Block-scaled FP6 (format 2 = E2M3, 3 = E3M2): one 32-element block of
// packed elements (24 bytes, element e at bits 6e .. 6e+5) per lane, lane half
// g holding block g of the instruction's 64 K (established on gfx950 with
// one-hot operands: every element of lane half g took block g's scale, with
// the value the packing gives).  K-tiles of 128 elements: 96 bytes of a row
// (kept in a 128-byte LDS row), blocks 2s and 2s+1 in step s; one scale word
// per row per k-tile.
template <int FA, int FB>
struct MmaMX6 {
    static constexpr bool kSparse = false, kScaled = true;
    static constexpr int kEsize = 1, kElemBits = 6, kAFrag = 24, kBFrag = 24, kKStep = 64;
    static constexpr int kBK = 128;
    static constexpr int kARowBytes = kBK * 6 / 8, kBRowBytes = kBK * 6 / 8;
    static constexpr int kScaleWords = kBK / 128;
    typedef f32x16 acc_t;
    typedef float out_t;
    // Operand bytes of lane half g: half 0 holds its block's bytes 0-15 in x and 16-23 in the low
    // half of z; half 1 its bytes 0-7 in the high half of z and 8-23 in x.
    __device__ __forceinline__ static i32x8 operand(const Frag<24> &f) {
        const bool h = (threadIdx.x & 32) != 0;
        return i32x8{h ? f.z[2] : f.x[0], h ? f.z[3] : f.x[1], h ? f.x[0] : f.x[2], h ? f.x[1] : f.x[3],
                     h ? f.x[2] : f.z[0], h ? f.x[3] : f.z[1], 0, 0};
    }
    __device__ __forceinline__ static acc_t mma_scaled(const Frag<24> &a, const Frag<24> &b, acc_t c, uint32_t sa,
                                                       uint32_t sb) {
        // the instruction reads six registers for FP6 operands; the last two are don't-cares
        const i32x8 A = operand(a), B = operand(b);
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, c, FA, FB, 0, (int)sa, 0, (int)sb);
    }
};

// Dense product (16- or 8-bit elements) with A stored M-contiguous (TA) and / or B stored
// N-contiguous (TB): same instruction, fragments read transposed.
template <class Base, bool TA, bool TB> struct Trans : Base {
    static constexpr bool kTransA = TA, kTransB = TB;
};

// Sparse instructions, A side: lane half g holds the compressed values of
// the g-th contiguous half of the instruction's dense K (in ascending order)
// and the index nibbles of those groups.  B side: the 64-byte K step of a B
// column splits into four 16-byte quarters; lane half g takes quarters g and
// 2 + g (registers 0-3 and 4-7).  This pairing was established on gfx950
// with one-hot products through this library (each compressed slot against
// an identity B, for all six index nibbles); it is what the parity tests
// against the oracle check on every run.
//
// Sparse fp16 / bf16: v_smfmac_f32_32x32x32_{f16,bf16}.  Per lane: 8
// compressed A values (16 B) = 16 dense K, 16 dense B values (32 B), and 16
// index bits (4 groups).  One index word covers the instruction's 32 dense K;
// lane half g takes its bits [16g, 16g + 16).
template <int DT> struct MmaSparse16 {
    static constexpr bool kSparse = true, kScaled = false;
    static constexpr int kScaleWords = 0;
    static constexpr int kEsize = 2, kAFrag = 16, kBFrag = 32, kKStep = 32;
    static constexpr int kBK = 64;                 // 64-byte compressed A rows, 128-byte B rows
    static constexpr int kARowBytes = kBK / 2 * kEsize, kBRowBytes = kBK * kEsize;
    static constexpr int kIdxWordsPerTile = kBK / 32;
    typedef f32x16 acc_t;
    typedef float out_t;
    __device__ __forceinline__ static constexpr int a_unit(int s, int g, int) { return 2 * s + g; }
    __device__ __forceinline__ static constexpr int b_unit(int s, int g, int h) { return 4 * s + g + 2 * h; }
    // Index words in LDS: the k-tile's two words of each row (one per step),
    // copied 4 bytes per lane, read by each lane with one 8-byte read (both
    // lane halves the same address, so the 32 rows of a read fill the 64 banks
    // once); lane half g takes bits [16g, 16g + 16) of the step's word.
    static constexpr int kIdxCopyBytes = 4;
    typedef i32x2 idx_t;
    __device__ __forceinline__ static idx_t load_idx(const uint8_t *row, int) {
        return *reinterpret_cast<const i32x2 *>(row);
    }
    __device__ __forceinline__ static uint32_t lane_idx(const idx_t &w, int s, int g) {
        return (uint32_t)w[s] >> (16 * g);
    }
    __device__ __forceinline__ static acc_t mma(const Frag<16> &a, const Frag<32> &b, acc_t c, uint32_t idx) {
        if constexpr (DT == DT_BF16)
            return __builtin_amdgcn_smfmac_f32_32x32x32_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                            __builtin_bit_cast(bf16x16, join(b)), c, (int)idx, 0, 0);
        else
            return __builtin_amdgcn_smfmac_f32_32x32x32_f16(__builtin_bit_cast(f16x8, a.v),
                                                           __builtin_bit_cast(f16x16, join(b)), c, (int)idx, 0, 0);
    }
};

// Sparse int8 / fp8 / bf8: v_smfmac_{i32,f32}_32x32x64_*.  Per lane: 16
// compressed A bytes = 32 dense K, 32 dense B bytes, 32 index bits (8 groups).
// The instruction's 64 dense K take two index words; lane half g takes word g.
template <int DT_A, int DT_B> struct MmaSparse8 {
    static constexpr bool kSparse = true, kScaled = false;
    static constexpr int kScaleWords = 0;
    static constexpr int kEsize = 1, kAFrag = 16, kBFrag = 32, kKStep = 64;
    static constexpr int kBK = 128;                // 64-byte compressed A rows, 128-byte B rows
    static constexpr int kARowBytes = kBK / 2, kBRowBytes = kBK;
    static constexpr int kIdxWordsPerTile = kBK / 32;
    static constexpr bool kInt = (DT_A == DT_I8);
    typedef typename std::conditional<kInt, i32x16, f32x16>::type acc_t;
    typedef typename std::conditional<kInt, int32_t, float>::type out_t;
    __device__ __forceinline__ static constexpr int a_unit(int s, int g, int) { return 2 * s + g; }
    __device__ __forceinline__ static constexpr int b_unit(int s, int g, int h) { return 4 * s + g + 2 * h; }
    // Index words in LDS: the k-tile's four words of each row (16 bytes),
    // copied 4 bytes per lane so that every copy pass is whole (a partly
    // filled pass would sit in a branch that splits the interleaved schedule
    // of the main loop), read by each lane with one 16-byte read, so 16
    // consecutive rows fill the 64 banks once; lane half g takes word g for
    // step 0 and word 2 + g for step 1.
    static constexpr int kIdxCopyBytes = 4;
    typedef i32x4 idx_t;
    __device__ __forceinline__ static idx_t load_idx(const uint8_t *row, int) {
        return *reinterpret_cast<const i32x4 *>(row);
    }
    __device__ __forceinline__ static uint32_t lane_idx(const idx_t &w, int s, int g) {
        return (uint32_t)(g ? w[2 * s + 1] : w[2 * s]);
    }
    __device__ __forceinline__ static acc_t mma(const Frag<16> &a, const Frag<32> &b, acc_t c, uint32_t idx) {
        if constexpr (kInt)
            return __builtin_amdgcn_smfmac_i32_32x32x64_i8(a.v, join(b), c, (int)idx, 0, 0);
        else if constexpr (DT_A == DT_E4M3 && DT_B == DT_E4M3)
            return __builtin_amdgcn_smfmac_f32_32x32x64_fp8_fp8(a.v, join(b), c, (int)idx, 0, 0);
        else if constexpr (DT_A == DT_E4M3 && DT_B == DT_E5M2)
            return __builtin_amdgcn_smfmac_f32_32x32x64_fp8_bf8(a.v, join(b), c, (int)idx, 0, 0);
        else if constexpr (DT_A == DT_E5M2 && DT_B == DT_E4M3)
            return __builtin_amdgcn_smfmac_f32_32x32x64_bf8_fp8(a.v, join(b), c, (int)idx, 0, 0);
        else
            return __builtin_amdgcn_smfmac_f32_32x32x64_bf8_bf8(a.v, join(b), c, (int)idx, 0, 0);
    }
};

}  // namespace mmac
