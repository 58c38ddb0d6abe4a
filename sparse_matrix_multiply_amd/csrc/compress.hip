// 4:2 compressor: dense A (M x K) -> compressed A (M x K/2) + index words.
//
// "CDNA3 sparse MFMA builtins", section "Structured sparsity (4:2 pattern)":
// walk each row along K in groups of four, find the two non-zero positions and
// pack those two values one after the other; the index names the positions,
// nibble p0 | (p1 << 2) with p0 < p1 (positions {0,2} -> 0x8, as the page's
// 0x88 / 0x8888 examples show).
//
// The work is a streaming copy, bound by HBM bandwidth: each thread owns one
// 16-byte chunk of a dense row (8 fp16/bf16 = 2 groups, or 16 one-byte
// elements = 4 groups), reads it with one 128-bit load and writes its 8
// compressed bytes with one 64-bit store; consecutive threads own consecutive
// chunks of a row, so both the loads and the stores of a wave are contiguous.
// The index bits of the 4 (two-byte types) or 2 (one-byte types) chunks that
// share one 32-bit word are gathered with lane shuffles and written by the
// first of those lanes.
#include <algorithm>

#include "device.h"
#include "launch.h"

namespace mmac {

// Nonzero test on raw bits: both signed zeros count as zero for the floating
// types; int8 has a single zero.  NaN is non-zero.
template <int DT>
__device__ __forceinline__ uint32_t nonzero(uint32_t x) {
    if constexpr (DT == DT_F16 || DT == DT_BF16) return (x & 0x7fffu) != 0u;
    else if constexpr (DT == DT_I8) return (x & 0xffu) != 0u;
    else return (x & 0x7fu) != 0u;
}

// Positions kept for a group whose non-zero mask is m (bit p = element p):
// the non-zero positions; if more than two, the two lowest (a violation); if
// fewer, topped up with the lowest positions not yet taken.  Returns the
// nibble p0 | (p1 << 2) and sets *viol.
__device__ __forceinline__ uint32_t pick_pair(uint32_t m, uint32_t *viol) {
    *viol = __builtin_popcount(m) > 2 ? 1u : 0u;
    uint32_t k = m;
    while (__builtin_popcount(k) < 2) k |= ~k & (k + 1u);   // add the lowest clear bit
    const uint32_t p0 = __builtin_ctz(k);
    const uint32_t p1 = __builtin_ctz(k & (k - 1u));
    return p0 | (p1 << 2);
}

template <int DT>
__global__ __launch_bounds__(256) void compress_kernel(CompressParams p, int cpr, int cpr_pad, int64_t total,
                                                       int64_t iters) {
    constexpr int ES = (DT == DT_F16 || DT == DT_BF16) ? 2 : 1;
    constexpr int PER = 16 / ES;         // elements per chunk
    constexpr int GROUPS = PER / 4;      // groups per chunk
    constexpr int LPW = 8 / GROUPS;      // chunks (lanes) per index word
    const int words = (p.K + 31) / 32;
    uint32_t bad = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t it = 0; it < iters; ++it) {
        const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x + it * stride;
        const int64_t row = t / cpr_pad;
        const int ch = (int)(t - row * cpr_pad);
        uint32_t bits = 0;
        if (t < total && ch < cpr) {
            const int e0 = ch * PER;
            const int ngroups = min(GROUPS, (p.K - e0) / 4);        // K % 4 == 0
            const uint8_t *src = p.A + row * p.a_pitch + (int64_t)e0 * ES;
            uint8_t *dst = p.Ac + row * p.ac_pitch + (int64_t)(e0 / 2) * ES;
            // chunk as 4 words; group q is word q (1-byte types) or words 2q, 2q+1 (2-byte types)
            uint32_t w[4] = {0, 0, 0, 0};
            if (ngroups == GROUPS) {
                const i32x4 v = *reinterpret_cast<const i32x4 *>(src);
                w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
            } else {
                for (int q = 0; q < ngroups * 4 * ES / 4; ++q) w[q] = reinterpret_cast<const uint32_t *>(src)[q];
            }
            uint32_t out[2] = {0, 0};     // 8 compressed bytes
#pragma unroll
            for (int q = 0; q < GROUPS; ++q) {
                if (q < ngroups) {
                    uint32_t e[4];
                    if constexpr (ES == 2) {
                        e[0] = w[2 * q] & 0xffffu; e[1] = w[2 * q] >> 16;
                        e[2] = w[2 * q + 1] & 0xffffu; e[3] = w[2 * q + 1] >> 16;
                    } else {
                        e[0] = w[q] & 0xffu; e[1] = (w[q] >> 8) & 0xffu;
                        e[2] = (w[q] >> 16) & 0xffu; e[3] = w[q] >> 24;
                    }
                    const uint32_t m = nonzero<DT>(e[0]) | nonzero<DT>(e[1]) << 1 | nonzero<DT>(e[2]) << 2 |
                                       nonzero<DT>(e[3]) << 3;
                    uint32_t viol;
                    const uint32_t nib = pick_pair(m, &viol);
                    bad += viol;
                    bits |= nib << (4 * q);
                    const uint32_t v0 = e[nib & 3u], v1 = e[nib >> 2];
                    if constexpr (ES == 2) out[q] = v0 | (v1 << 16);
                    else out[q / 2] |= (v0 | (v1 << 8)) << (16 * (q % 2));
                }
            }
            if (ngroups == GROUPS) {
                *reinterpret_cast<i32x2 *>(dst) = i32x2{(int)out[0], (int)out[1]};
            } else {
                // ngroups * 2 elements of ES bytes: a whole number of 2-byte (1-byte types) or
                // 4-byte (2-byte types) pieces
                if constexpr (ES == 2) {
                    for (int q = 0; q < ngroups; ++q) reinterpret_cast<uint32_t *>(dst)[q] = out[q];
                } else {
                    for (int q = 0; q < ngroups; ++q)
                        reinterpret_cast<uint16_t *>(dst)[q] = (uint16_t)(out[q / 2] >> (16 * (q % 2)));
                }
            }
        }
        // gather the index bits of the LPW chunks of one word (whole wave takes part)
        uint32_t word = bits << (4 * GROUPS * (ch % LPW));
        word |= __shfl_xor(word, 1);
        if constexpr (LPW == 4) word |= __shfl_xor(word, 2);
        if (t < total && (ch % LPW) == 0 && ch / LPW < words)
            p.idx[row * p.idx_pitch + ch / LPW] = word;
    }
    if (p.bad) {
        // one atomic per wave that saw a violation
        for (int off = 32; off > 0; off >>= 1) bad += __shfl_xor(bad, off);
        if ((threadIdx.x & 63) == 0 && bad) atomicAdd(p.bad, bad);
    }
}

hipError_t launch_compress(int dt, CompressParams p, hipStream_t s) {
    const int es = (dt == DT_F16 || dt == DT_BF16) ? 2 : 1;
    const int lpw = es == 2 ? 4 : 2;
    const int cpr = (int)(((int64_t)p.K * es + 15) / 16);
    const int cpr_pad = (cpr + lpw - 1) / lpw * lpw;
    const int64_t total = (int64_t)p.M * cpr_pad;
    const int64_t max_blocks = 256 * 64;          // enough waves to cover the chip many times over
    const int64_t blocks = std::min<int64_t>((total + 255) / 256, max_blocks);
    const int64_t iters = (total + blocks * 256 - 1) / (blocks * 256);
    const dim3 grid((unsigned)blocks), block(256);
    switch (dt) {
    case DT_F16: hipLaunchKernelGGL(compress_kernel<DT_F16>, grid, block, 0, s, p, cpr, cpr_pad, total, iters); break;
    case DT_BF16: hipLaunchKernelGGL(compress_kernel<DT_BF16>, grid, block, 0, s, p, cpr, cpr_pad, total, iters); break;
    case DT_I8: hipLaunchKernelGGL(compress_kernel<DT_I8>, grid, block, 0, s, p, cpr, cpr_pad, total, iters); break;
    case DT_E4M3: hipLaunchKernelGGL(compress_kernel<DT_E4M3>, grid, block, 0, s, p, cpr, cpr_pad, total, iters); break;
    case DT_E5M2: hipLaunchKernelGGL(compress_kernel<DT_E5M2>, grid, block, 0, s, p, cpr, cpr_pad, total, iters); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mmac
