// Tiled GEMM kernel shared by the dense (MFMA) and 4:2-sparse (SMFMAC) paths.
//
// One workgroup computes a BM x BN tile of D; its WM x WN waves each own a
// (BM/WM) x (BN/WN) sub-tile made of 32 x 32 instruction tiles.  K is walked
// in k-tiles of Op::kBK dense elements (one 128-byte LDS row for B; 128 or 64
// bytes for A, which is half as long when compressed).  Each k-tile of A and B
// is copied from HBM straight into LDS by buffer loads with an LDS
// destination (no register staging), into one of two LDS stages, while the
// waves run the matrix instructions on the other stage.  Rows past M and
// columns past N read as zero through the buffer descriptor's range check; a
// ragged last k-tile is filled through registers with explicit zero masking.
//
// The multiply-accumulate follows "CDNA dense MFMA builtins", section
// "Naming convention" (each instruction adds one K panel; the kernel loops
// over K), and for sparse A "CDNA3 sparse MFMA builtins", section "Structured
// sparsity (4:2 pattern)".  The epilogue maps (lane, register) to (i, j) with
// the one-block 32 x 32 accumulator layout of "CDNA dense MFMA builtins",
// "Accumulator layout": i = 8*floor(G/4) + 4*floor(L/32) + (G mod 4),
// j = L mod 32.
#pragma once

#include <type_traits>

#include "device.h"
#include "launch.h"

namespace mmac {

// Workgroup -> output tile.  Workgroups are dealt to the 8 XCDs round-robin
// (workgroup w runs on XCD w mod 8), so first give each XCD a contiguous run of
// tile numbers, then walk tile numbers in groups of `group_m` tile rows,
// column by column, so the tiles an XCD runs at the same time share A row
// panels and B column panels in that XCD's L2.
__device__ __forceinline__ void tile_coords(int wg, const GemmParams &p, int &tm, int &tn) {
    const int T = p.tiles_m * p.tiles_n;
    const int x = wg & 7, local = wg >> 3, q = T >> 3, r = T & 7;
    const int t = x * q + (x < r ? x : r) + local;
    const int per_group = p.group_m * p.tiles_n;
    const int grp = t / per_group;
    const int first = grp * p.group_m;
    const int gsz = min(p.tiles_m - first, p.group_m);
    const int in = t - grp * per_group;
    tm = first + in % gsz;
    tn = in / gsz;
}

// s_waitcnt with vmcnt = 0 (expcnt and lgkmcnt left at their maxima).
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// One fragment from LDS: 16-byte units u0 (and u1 for 32-byte fragments) of a tile.
template <int BYTES>
__device__ __forceinline__ void lds_frag(Frag<BYTES> &f, const uint8_t *base, uint32_t u0, uint32_t u1) {
    if constexpr (BYTES == 16) {
        f.v = *reinterpret_cast<const i32x4 *>(base + swz(u0) * 16);
    } else {
        f.lo = *reinterpret_cast<const i32x4 *>(base + swz(u0) * 16);
        f.hi = *reinterpret_cast<const i32x4 *>(base + swz(u1) * 16);
    }
}

// 16 bytes of one row starting at element e0 of that row, keeping only the
// elements below `limit` (the rest become zero).  Used for the ragged k-tile.
template <int ESIZE>
__device__ __forceinline__ i32x4 masked_unit(rsrc_t r, uint32_t off, int e0, int limit) {
    constexpr int PER = 16 / ESIZE;
    if (e0 + PER <= limit) return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    i32x4 v = {0, 0, 0, 0};
    if (e0 >= limit) return v;
    uint32_t w[4] = {0, 0, 0, 0};
    for (int e = 0; e < PER; ++e) {
        if (e0 + e < limit) {
            uint32_t x;
            if constexpr (ESIZE == 2) x = __builtin_amdgcn_raw_buffer_load_b16(r, off + 2 * e, 0, 0);
            else x = __builtin_amdgcn_raw_buffer_load_b8(r, off + e, 0, 0);
            w[(e * ESIZE) / 4] |= x << (8 * ((e * ESIZE) % 4));
        }
    }
    v[0] = (int)w[0]; v[1] = (int)w[1]; v[2] = (int)w[2]; v[3] = (int)w[3];
    return v;
}

template <class Op, int BM, int BN, int WM, int WN>
struct TiledGemm {
    typedef typename Op::acc_t acc_t;
    typedef typename Op::out_t out_t;
    static constexpr int NT = WM * WN * 64;
    static constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 tiles");
    static constexpr int AW = Op::kARowBytes / 16, BW = Op::kBRowBytes / 16;  // 16-byte units per LDS row
    static_assert(AW == 4 || AW == 8, "LDS rows of 64 or 128 bytes");
    static_assert(BW == 8, "B LDS rows of 128 bytes");
    static constexpr int AQ = BM * AW / NT, BQ = BN * BW / NT;                  // DMA units per thread
    static_assert(AQ * NT == BM * AW && BQ * NT == BN * BW, "tile not a whole number of DMA passes");
    static constexpr int A_BYTES = BM * AW * 16, B_BYTES = BN * BW * 16, STAGE = A_BYTES + B_BYTES;
    static constexpr int STEPS = Op::kBK / Op::kKStep;
    static constexpr int IW = Op::kSparse ? Op::kBK / 32 : 1;                   // index words per k-tile row

    const GemmParams &p;
    int tid, wave, g, l32, wm, wn, row0, col0, arows, bcols;
    rsrc_t ra, rb, rx;
    uint32_t a_off[AQ], b_off[BQ];   // byte offset (k-tile 0) of the unit copied in DMA pass q
    acc_t acc[TM][TN];

    __device__ __forceinline__ TiledGemm(const GemmParams &p_) : p(p_) {
        tid = threadIdx.x;
        const int lane = tid & 63;
        wave = tid >> 6;
        g = lane >> 5;
        l32 = lane & 31;
        wm = wave / WN;
        wn = wave % WN;
        int tm, tn;
        tile_coords(blockIdx.x, p, tm, tn);
        row0 = tm * BM;
        col0 = tn * BN;
        arows = min(BM, p.M - row0);
        bcols = min(BN, p.N - col0);
        ra = make_rsrc(p.A + (int64_t)row0 * p.a_pitch, (uint32_t)(arows * p.a_pitch));
        rb = make_rsrc(p.B + (int64_t)col0 * p.b_pitch, (uint32_t)(bcols * p.b_pitch));
        if constexpr (Op::kSparse)
            rx = make_rsrc(p.idx + (int64_t)row0 * p.idx_pitch, (uint32_t)(arows * p.idx_pitch * 4));
#pragma unroll
        for (int q = 0; q < AQ; ++q) {
            const uint32_t L = swz(tid + q * NT);
            a_off[q] = (L / AW) * (uint32_t)p.a_pitch + (L % AW) * 16;
        }
#pragma unroll
        for (int q = 0; q < BQ; ++q) {
            const uint32_t L = swz(tid + q * NT);
            b_off[q] = (L / BW) * (uint32_t)p.b_pitch + (L % BW) * 16;
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = acc_t{};
    }

    // Copy k-tile kt of A and B into the LDS stage `st` (asynchronous; rows past M / N read as zero).
    __device__ __forceinline__ void dma(uint8_t *st, int kt) {
        const uint32_t ka = kt * Op::kARowBytes, kb = kt * Op::kBRowBytes;
#pragma unroll
        for (int q = 0; q < AQ; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(st + (q * NT + wave * 64) * 16), 16,
                                                     a_off[q] + ka, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < BQ; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(st + A_BYTES + (q * NT + wave * 64) * 16), 16,
                                                     b_off[q] + kb, 0, 0, 0);
    }

    // The ragged last k-tile, filled through registers with elements past K set to zero.
    __device__ __forceinline__ void fill_masked(uint8_t *st, int kt) {
        const int climit = Op::kSparse ? p.K / 2 : p.K;      // elements of A per row
#pragma unroll
        for (int q = 0; q < AQ; ++q) {
            const uint32_t P = tid + q * NT, L = swz(P);
            const int e0 = (kt * Op::kARowBytes + (int)(L % AW) * 16) / Op::kEsize;
            *reinterpret_cast<i32x4 *>(st + P * 16) =
                masked_unit<Op::kEsize>(ra, a_off[q] + kt * Op::kARowBytes, e0, climit);
        }
#pragma unroll
        for (int q = 0; q < BQ; ++q) {
            const uint32_t P = tid + q * NT, L = swz(P);
            const int e0 = (kt * Op::kBRowBytes + (int)(L % BW) * 16) / Op::kEsize;
            *reinterpret_cast<i32x4 *>(st + A_BYTES + P * 16) =
                masked_unit<Op::kEsize>(rb, b_off[q] + kt * Op::kBRowBytes, e0, p.K);
        }
    }

    // Sparse index words of this lane's rows for k-tile kt.
    __device__ __forceinline__ void load_idx(uint32_t (&w)[TM][IW], int kt) {
        if constexpr (Op::kSparse) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const uint32_t r = wm * WTM + i * 32 + l32;
#pragma unroll
                for (int q = 0; q < IW; ++q)
                    w[i][q] = __builtin_amdgcn_raw_buffer_load_b32(rx, (r * (uint32_t)p.idx_pitch + kt * IW + q) * 4,
                                                                   0, 0);
            }
        }
    }

    typedef Frag<Op::kAFrag> FragA;
    typedef Frag<Op::kBFrag> FragB;

    // Fragments of step s of the k-tile held in LDS stage `st`.
    __device__ __forceinline__ void load_frags(FragA (&a)[TM], FragB (&b)[TN], const uint8_t *st, int s) {
        const uint8_t *sa = st, *sb = st + A_BYTES;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const uint32_t r = (wm * WTM + i * 32 + l32) * AW;
            lds_frag(a[i], sa, r + Op::a_unit(s, g, 0), r + Op::a_unit(s, g, 1));
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const uint32_t r = (wn * WTN + j * 32 + l32) * BW;
            lds_frag(b[j], sb, r + Op::b_unit(s, g, 0), r + Op::b_unit(s, g, 1));
        }
    }

    // The TM x TN matrix instructions of step s.
    __device__ __forceinline__ void mma_step(const FragA (&a)[TM], const FragB (&b)[TN], const uint32_t (&w)[TM][IW],
                                             int s) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            uint32_t ix = 0;
            if constexpr (Op::kSparse) ix = Op::lane_idx(w[i], s, g);
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = Op::mma(a[i], b[j], acc[i][j], ix);
        }
    }

    // D = alpha * acc + beta * C, element (i, j) of a 32 x 32 tile being
    // register G of lane L with i = 8*floor(G/4) + 4*floor(L/32) + (G mod 4),
    // j = L mod 32 (lanes 0-31 and 32-63 each write 32 consecutive floats of a row).
    __device__ __forceinline__ void epilogue() {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int col = col0 + wn * WTN + j * 32 + l32;
#pragma unroll
                for (int G = 0; G < 16; ++G) {
                    const int row = row0 + wm * WTM + i * 32 + 8 * (G / 4) + 4 * g + (G % 4);
                    if (row < p.M && col < p.N) {
                        out_t *d = reinterpret_cast<out_t *>(p.D) + (int64_t)row * p.ldd + col;
                        if constexpr (std::is_same<out_t, float>::value) {
                            float v = p.alpha * acc[i][j][G];
                            if (p.use_c)
                                v = fmaf(p.beta, reinterpret_cast<const float *>(p.C)[(int64_t)row * p.ldc + col], v);
                            *d = v;
                        } else {
                            uint32_t v = (uint32_t)p.ialpha * (uint32_t)acc[i][j][G];
                            if (p.use_c)
                                v += (uint32_t)p.ibeta *
                                     (uint32_t)reinterpret_cast<const int32_t *>(p.C)[(int64_t)row * p.ldc + col];
                            *d = (int32_t)v;
                        }
                    }
                }
            }
        }
    }
};

template <class Op, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM *WN * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_tiled_kernel(GemmParams p) {
    typedef TiledGemm<Op, BM, BN, WM, WN> T;
    constexpr int IW = T::IW, TM = T::TM;
    __shared__ __attribute__((aligned(16))) uint8_t st0[T::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st1[T::STAGE];
    T t(p);

    const int nk = p.K / Op::kBK;                        // whole k-tiles
    const int nkt = nk + (p.K > nk * Op::kBK ? 1 : 0);   // plus a ragged one
    constexpr int STEPS = T::STEPS;
    static_assert(STEPS % 2 == 0, "fragment double buffering assumes an even number of steps");
    uint32_t ixc[TM][IW], ixn[TM][IW];
    typename T::FragA a[2][TM];
    typename T::FragB b[2][T::TN];

    // Software pipeline: the fragments of step s + 1 are read from LDS while the
    // matrix instructions of step s run; the block barrier that hands over the
    // next LDS stage sits before the last step's instructions, so the first
    // reads of the next k-tile overlap them.  The copy of k-tile kt + 1 into the
    // other stage is in flight during the whole of k-tile kt.
    if (nkt > 0) {
        if (0 < nk) t.dma(st0, 0);
        else t.fill_masked(st0, 0);
        t.load_idx(ixc, 0);
        wait_vmem_all();
        __syncthreads();
        t.load_frags(a[0], b[0], st0, 0);
    }
    for (int kt = 0; kt < nkt; ++kt) {
        const uint8_t *cur = (kt & 1) ? st1 : st0;
        uint8_t *nxt = (kt & 1) ? st0 : st1;
        if (kt + 1 < nkt) {
            if (kt + 1 < nk) t.dma(nxt, kt + 1);
            else t.fill_masked(nxt, kt + 1);
            t.load_idx(ixn, kt + 1);
        }
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            const int cb = s & 1;
            if (s + 1 < STEPS) {
                t.load_frags(a[cb ^ 1], b[cb ^ 1], cur, s + 1);
            } else {
                wait_vmem_all();
                __syncthreads();
                if (kt + 1 < nkt) t.load_frags(a[cb ^ 1], b[cb ^ 1], nxt, 0);
            }
            t.mma_step(a[cb], b[cb], ixc, s);
        }
        if constexpr (Op::kSparse) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int q = 0; q < IW; ++q) ixc[i][q] = ixn[i][q];
        }
    }
    t.epilogue();
}

}  // namespace mmac
