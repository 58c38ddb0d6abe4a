// 4:2 compressor: dense A (M x K) -> compressed A (M x K/2) + index words,
// optionally after magnitude pruning to the 4:2 pattern.
//
// "CDNA3 sparse MFMA builtins", section "Structured sparsity (4:2 pattern)":
// walk each row along K in groups of four, find the two non-zero positions and
// pack those two values one after the other; the index names the positions,
// nibble p0 | (p1 << 2) with p0 < p1 (positions {0,2} -> 0x8, as the page's
// 0x88 / 0x8888 examples show).
//
// The work is a streaming copy, bound by HBM bandwidth, so the per-element
// work is kept to a few instructions: each thread owns one 16-byte chunk of a
// dense row (8 two-byte or 16 one-byte elements = 2 or 4 groups), reads it
// with one 128-bit load, finds the non-zero masks of its groups with packed
// word arithmetic, looks the kept pair up in a 16-entry table, gathers the
// kept elements with byte permutes, and writes its 8 compressed bytes with one
// 64-bit store.  Consecutive threads own consecutive chunks of a row (the grid
// is chunks x rows), so both the loads and the stores of a wave are
// contiguous.  The index bits of the 4 (two-byte types) or 2 (one-byte types)
// chunks that share a 32-bit word are gathered with lane shuffles and written
// by the first of those lanes.
//
// With pruning, the kept pair of a group is the two largest magnitudes
// (ties to the lower position) instead of the non-zeros; everything else is
// the same pass, so a dense A goes to the compressed form in one read.
#include <algorithm>

#include "device.h"
#include "launch.h"

namespace mmac {

// Kept positions for a group whose non-zero mask is m (bit p = element p):
// the non-zero positions; if more than two, the two lowest; if fewer, topped
// up with the lowest positions not yet taken.  Returns p0 | (p1 << 2).
constexpr uint32_t kept_pair(uint32_t m) {
    uint32_t k = m;
    while (__builtin_popcount(k) < 2) k |= ~k & (k + 1u);   // add the lowest clear bit
    return (uint32_t)__builtin_ctz(k) | ((uint32_t)__builtin_ctz(k & (k - 1u)) << 2);
}
constexpr uint64_t pair_table() {
    uint64_t t = 0;
    for (uint32_t m = 0; m < 16; ++m) t |= (uint64_t)kept_pair(m) << (4 * m);
    return t;
}
constexpr uint64_t kPairTable = pair_table();
// masks with more than two non-zeros: 0b0111, 0b1011, 0b1101, 0b1110, 0b1111
constexpr uint32_t kViolations = (1u << 7) | (1u << 11) | (1u << 13) | (1u << 14) | (1u << 15);

// Non-zero mask of the 4-element group held in one word (one-byte types):
// floating types treat both signed zeros as zero (bit 7 ignored), int8 has one zero.
template <int DT>
__device__ __forceinline__ uint32_t group_mask8(uint32_t w) {
    uint32_t nz;
    if constexpr (DT == DT_I8) nz = (((w & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w) & 0x80808080u;
    else nz = ((w & 0x7f7f7f7fu) + 0x7f7f7f7fu) & 0x80808080u;
    return ((nz >> 7) & 1u) | ((nz >> 14) & 2u) | ((nz >> 21) & 4u) | ((nz >> 28) & 8u);
}

// Non-zero mask of the 4-element group held in two words (two-byte floating types).
__device__ __forceinline__ uint32_t group_mask16(uint32_t w0, uint32_t w1) {
    const uint32_t n0 = ((w0 & 0x7fff7fffu) + 0x7fff7fffu) & 0x80008000u;
    const uint32_t n1 = ((w1 & 0x7fff7fffu) + 0x7fff7fffu) & 0x80008000u;
    return ((n0 >> 15) & 1u) | ((n0 >> 30) & 2u) | ((n1 >> 13) & 4u) | ((n1 >> 28) & 8u);
}

// Magnitude pruning: sort key of element p of a group of two-byte elements
// (raw bits e).  The magnitude bits of these sign-magnitude formats order like
// the magnitudes; every NaN maps to one value just above infinity (so all NaNs
// tie and beat every number).  The low two bits make the keys distinct, the
// lower position winning a tie.  (The one-byte types use top2_nibbles8 below;
// there E4M3's only NaN code is already the largest magnitude.)
template <int DT>
__device__ __forceinline__ uint32_t mag_key(uint32_t e, int p) {
    static_assert(DT == DT_F16 || DT == DT_BF16, "two-byte types");
    const uint32_t m = min(e & 0x7fffu, DT == DT_F16 ? 0x7c01u : 0x7f81u);
    return (m << 2) | (uint32_t)(3 - p);
}

// Mask of the two largest of four distinct keys: element p is kept when fewer
// than two keys exceed its own.
__device__ __forceinline__ uint32_t top2_mask(uint32_t k0, uint32_t k1, uint32_t k2, uint32_t k3) {
    const uint32_t a = k1 > k0, b = k2 > k0, c = k3 > k0, d = k2 > k1, e = k3 > k1, f = k3 > k2;
    const uint32_t r0 = a + b + c, r1 = 1 - a + d + e, r2 = 2 - b - d + f, r3 = 3 - c - e - f;
    return (uint32_t)(r0 < 2) | ((uint32_t)(r1 < 2) << 1) | ((uint32_t)(r2 < 2) << 2) | ((uint32_t)(r3 < 2) << 3);
}

// Kept-position mask of group q of the chunk w: the non-zeros (plain
// compression) or the two largest magnitudes (PRUNE).
template <int DT, bool PRUNE>
__device__ __forceinline__ uint32_t keep_mask(const uint32_t (&w)[4], int q, uint32_t nonzero) {
    if constexpr (!PRUNE) {
        return nonzero;
    } else if constexpr (DT == DT_F16 || DT == DT_BF16) {
        const uint32_t lo = w[2 * q], hi = w[2 * q + 1];
        return top2_mask(mag_key<DT>(lo & 0xffffu, 0), mag_key<DT>(lo >> 16, 1), mag_key<DT>(hi & 0xffffu, 2),
                         mag_key<DT>(hi >> 16, 3));
    } else {
        static_assert(DT == DT_F16 || DT == DT_BF16, "one-byte types prune with top2_nibbles8");
        return 0;
    }
}

// Packed form of the pruning rank for the one-byte types: two groups at once,
// one per 16-bit half of each register, with v_pk_max/min_u16.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_max(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ uint32_t pk_min(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}

// Magnitudes of the four one-byte elements of a word, byte for byte: fp8
// drops the sign; int8 takes |v| (one's complement plus one where negative; no
// byte carries, -128 -> 0x80).
template <int DT>
__device__ __forceinline__ uint32_t mag_bytes(uint32_t w) {
    if constexpr (DT == DT_I8) {
        const uint32_t s = (w >> 7) & 0x01010101u;
        return (w ^ (s * 0xffu)) + s;
    } else {
        return w & 0x7f7f7f7fu;
    }
}

// Kept-pair nibbles of two groups of four one-byte elements (words wa, wb):
// nib(wa) | nib(wb) << 16.  Key of element p = magnitude << 2 | (3 - p) in a
// 16-bit half (E5M2 NaNs first folded to one code above infinity); the two
// largest of four keys are the larger pair winner and the larger of the other
// winner and both losers.
template <int DT>
__device__ __forceinline__ uint32_t top2_nibbles8(uint32_t wa, uint32_t wb) {
    const uint32_t ma = mag_bytes<DT>(wa), mb = mag_bytes<DT>(wb);
    uint32_t k[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        // [ma byte e, 0, mb byte e, 0]
        uint32_t m = __builtin_amdgcn_perm(mb, ma, (uint32_t)e | (0x0cu << 8) | ((4u + e) << 16) | (0x0cu << 24));
        if constexpr (DT == DT_E5M2) m = pk_min(m, 0x007d007du);
        k[e] = (m << 2) | ((3u - e) * 0x00010001u);
    }
    const uint32_t m1 = pk_max(k[0], k[1]), n1 = pk_min(k[0], k[1]);
    const uint32_t m2 = pk_max(k[2], k[3]), n2 = pk_min(k[2], k[3]);
    const uint32_t first = pk_max(m1, m2), second = pk_max(pk_min(m1, m2), pk_max(n1, n2));
    const uint32_t pf = 0x00030003u - (first & 0x00030003u), ps = 0x00030003u - (second & 0x00030003u);
    return pk_min(pf, ps) | (pk_max(pf, ps) << 2);
}

template <int DT, bool PRUNE>
__global__ __launch_bounds__(256) void compress_kernel(CompressParams p, int cpr) {
    constexpr int ES = (DT == DT_F16 || DT == DT_BF16) ? 2 : 1;
    constexpr int PER = 16 / ES;         // elements per chunk
    constexpr int GROUPS = PER / 4;      // groups per chunk
    constexpr int LPW = 8 / GROUPS;      // chunks (lanes) per index word
    const int ch = blockIdx.x * 256 + threadIdx.x;      // chunk within the row
    const int words = (p.K + 31) / 32;
    const int e0 = ch * PER;
    const int ngroups = ch < cpr ? min(GROUPS, (p.K - e0) / 4) : 0;   // K % 4 == 0
    uint32_t bad = 0;
    for (int row = blockIdx.y; row < p.M; row += gridDim.y) {
        const uint8_t *src = p.A + (int64_t)row * p.a_pitch + (int64_t)e0 * ES;
        uint8_t *dst = p.Ac + (int64_t)row * p.ac_pitch + (int64_t)(e0 / 2) * ES;
        uint32_t bits = 0;
        if (ngroups > 0) {
            uint32_t w[4] = {0, 0, 0, 0};   // the chunk; group q is word q (1-byte) or words 2q, 2q+1
            if (ngroups == GROUPS) {
                const i32x4 v = *reinterpret_cast<const i32x4 *>(src);
                w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
            } else {
                for (int q = 0; q < ngroups * ES; ++q) w[q] = reinterpret_cast<const uint32_t *>(src)[q];
            }
            uint32_t out[2] = {0, 0};     // 8 compressed bytes
            uint32_t nib[4];
            if constexpr (PRUNE && ES == 1) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t nn = top2_nibbles8<DT>(w[2 * h], w[2 * h + 1]);
                    nib[2 * h] = nn & 0xfu;
                    nib[2 * h + 1] = nn >> 16;
                }
            }
#pragma unroll
            for (int q = 0; q < GROUPS; ++q) {
                const uint32_t m = (ES == 2) ? group_mask16(w[2 * q], w[2 * q + 1]) : group_mask8<DT>(w[q]);
                if constexpr (!(PRUNE && ES == 1))
                    nib[q] = (uint32_t)(kPairTable >> (4 * keep_mask<DT, PRUNE>(w, q, m))) & 0xfu;
                if (q < ngroups) {
                    bad += (kViolations >> m) & 1u;
                    bits |= nib[q] << (4 * q);
                }
            }
            if constexpr (ES == 2) {
                // group q -> one word: [half p0, half p1] picked from the 8 bytes (w[2q+1]:w[2q])
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const uint32_t a = 2 * (nib[q] & 3u), b = 2 * (nib[q] >> 2);
                    out[q] = __builtin_amdgcn_perm(w[2 * q + 1], w[2 * q], a | ((a + 1) << 8) | (b << 16) | ((b + 1) << 24));
                }
            } else {
                // groups 2h, 2h+1 -> one word: [g0.p0, g0.p1, g1.p0, g1.p1] picked from (w[2h+1]:w[2h])
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t n0 = nib[2 * h], n1 = nib[2 * h + 1];
                    const uint32_t sel = (n0 & 3u) | ((n0 >> 2) << 8) | ((4u + (n1 & 3u)) << 16) | ((4u + (n1 >> 2)) << 24);
                    out[h] = __builtin_amdgcn_perm(w[2 * h + 1], w[2 * h], sel);
                }
            }
            if (ngroups == GROUPS) {
                *reinterpret_cast<i32x2 *>(dst) = i32x2{(int)out[0], (int)out[1]};
            } else if constexpr (ES == 2) {
                for (int q = 0; q < ngroups; ++q) reinterpret_cast<uint32_t *>(dst)[q] = out[q];
            } else {
                for (int q = 0; q < ngroups; ++q)
                    reinterpret_cast<uint16_t *>(dst)[q] = (uint16_t)(out[q / 2] >> (16 * (q % 2)));
            }
        }
        // gather the index bits of the LPW chunks of one word (the whole wave takes part)
        uint32_t word = bits << (4 * GROUPS * (ch % LPW));
        word |= __shfl_xor(word, 1);
        if constexpr (LPW == 4) word |= __shfl_xor(word, 2);
        if ((ch % LPW) == 0 && ch / LPW < words) p.idx[(int64_t)row * p.idx_pitch + ch / LPW] = word;
    }
    if (p.bad) {
        // one atomic per wave that saw a violation
        for (int off = 32; off > 0; off >>= 1) bad += __shfl_xor(bad, off);
        if ((threadIdx.x & 63) == 0 && bad) atomicAdd(p.bad, bad);
    }
}

template <bool PRUNE>
static hipError_t launch_mode(int dt, const CompressParams &p, hipStream_t s) {
    const int es = (dt == DT_F16 || dt == DT_BF16) ? 2 : 1;
    const int cpr = (int)(((int64_t)p.K * es + 15) / 16);      // 16-byte chunks per row
    const dim3 grid((unsigned)((cpr + 255) / 256), (unsigned)std::min(p.M, 65535)), block(256);
    switch (dt) {
    case DT_F16: hipLaunchKernelGGL((compress_kernel<DT_F16, PRUNE>), grid, block, 0, s, p, cpr); break;
    case DT_BF16: hipLaunchKernelGGL((compress_kernel<DT_BF16, PRUNE>), grid, block, 0, s, p, cpr); break;
    case DT_I8: hipLaunchKernelGGL((compress_kernel<DT_I8, PRUNE>), grid, block, 0, s, p, cpr); break;
    case DT_E4M3: hipLaunchKernelGGL((compress_kernel<DT_E4M3, PRUNE>), grid, block, 0, s, p, cpr); break;
    case DT_E5M2: hipLaunchKernelGGL((compress_kernel<DT_E5M2, PRUNE>), grid, block, 0, s, p, cpr); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_compress(int dt, CompressParams p, bool prune, hipStream_t s) {
    return prune ? launch_mode<true>(dt, p, s) : launch_mode<false>(dt, p, s);
}

}  // namespace mmac
