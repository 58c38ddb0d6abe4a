// Tiled GEMM kernel shared by the dense (MFMA) and 4:2-sparse (SMFMAC) paths.
//
// One workgroup computes a BM x BN tile of D; its WM x WN waves each own a
// (BM/WM) x (BN/WN) sub-tile made of 32 x 32 instruction tiles.  K is walked
// in k-tiles of Op::kBK dense elements, from a per-tile starting k-tile (see
// the kernel) with wrap-around.  Each k-tile of A (or compressed A),
// B and, for sparse A, the index words is copied from memory straight into
// LDS by buffer loads with an LDS destination (no register staging).  There
// are STAGES LDS stages: while the waves run the matrix instructions of
// k-tile kt, the copies of k-tiles kt+1 .. kt+STAGES-1 are in flight, and the
// wait at the end of an iteration only drains the copy of k-tile kt+1
// (counted vmcnt), so several k-tiles' worth of memory latency is hidden.
// Rows past M and columns past N read as zero through the buffer descriptor's
// range check; a ragged last k-tile is filled through registers with explicit
// zero masking.
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

// Workgroup -> (output tile, K range).  Workgroups are dealt to the 8 XCDs
// round-robin (workgroup w runs on XCD w mod 8), so first give each XCD a
// contiguous run of unit numbers (the K ranges of one tile are consecutive
// units, so they normally share an XCD and its L2), then walk tile numbers in
// groups of `group_m` tile rows, column by column, so the tiles an XCD runs at
// the same time share A row panels and B column panels in that XCD's L2.
__device__ __forceinline__ void tile_coords(int wg, const GemmParams &p, int &tm, int &tn, int &split) {
    const int U = p.tiles_m * p.tiles_n * p.splits;
    const int x = wg & 7, local = wg >> 3, q = U >> 3, r = U & 7;
    const int u = x * q + (x < r ? x : r) + local;
    const int t = u / p.splits;
    split = u - t * p.splits;
    const int per_group = p.group_m * p.tiles_n;
    const int grp = t / per_group;
    const int first = grp * p.group_m;
    const int gsz = min(p.tiles_m - first, p.group_m);
    const int in = t - grp * per_group;
    tm = first + in % gsz;
    tn = in / gsz;
}

// s_waitcnt encoding on gfx9: vmcnt in bits [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8].  Waits for vmcnt <= VM and lgkmcnt == 0.
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    __builtin_amdgcn_sched_barrier(0);   // keep the instruction order across the wait
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));
    asm volatile("" ::: "memory");
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every outstanding copy); the waits that are needed are explicit.
__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// One fragment from LDS: 16-byte units u0 (and u1 for 32-byte fragments) of a
// tile with W units per row.
template <int W, int BYTES>
__device__ __forceinline__ void lds_frag(Frag<BYTES> &f, const uint8_t *base, uint32_t u0, uint32_t u1) {
    if constexpr (BYTES == 16) {
        f.v = *reinterpret_cast<const i32x4 *>(base + swz<W>(u0) * 16);
    } else {
        f.lo = *reinterpret_cast<const i32x4 *>(base + swz<W>(u0) * 16);
        f.hi = *reinterpret_cast<const i32x4 *>(base + swz<W>(u1) * 16);
    }
}

// Instruction classes for __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100;

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

// Wait until at most n * LPT copy instructions of this wave are outstanding
// (and every LDS access has completed); n is in [0, MAXN].
template <int LPT, int MAXN>
__device__ __forceinline__ void wait_copies(int n) {
    if constexpr (MAXN <= 0) {
        wait_vm_lgkm0<0>();
    } else {
        if (n >= MAXN) wait_vm_lgkm0<MAXN * LPT>();
        else wait_copies<LPT, MAXN - 1>(n);
    }
}

// Bits per element of an operand (packed FP4: 4, packed FP6: 6).
template <class O, class = void> struct ElemBits { static constexpr int value = 8 * O::kEsize; };
template <class O> struct ElemBits<O, std::void_t<decltype(O::kElemBits)>> { static constexpr int value = O::kElemBits; };

// Operands stored with M (A) or N (B) contiguous instead of K (16- and 8-bit types).
template <class O, class = void> struct TransOf { static constexpr bool a = false, b = false; };
template <class O> struct TransOf<O, std::void_t<decltype(O::kTransA)>> {
    static constexpr bool a = O::kTransA, b = O::kTransB;
};

// Bytes of index words one copy lane moves (sparse A only).
template <class O>
constexpr int idx_copy_bytes() {
    if constexpr (O::kSparse) return O::kIdxCopyBytes;
    else return 4;
}

template <class Op, int BM, int BN, int WM, int WN, int STAGES_>
struct TiledGemm {
    typedef typename Op::acc_t acc_t;
    typedef typename Op::out_t out_t;
    static constexpr int NW = WM * WN, NT = NW * 64, STAGES = STAGES_;
    static constexpr int STEPS = Op::kBK / Op::kKStep;
    static constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 tiles");
    // Bytes of a row that one k-tile covers (ARB, BRB) and 16-byte units per LDS
    // row (AW, BW): the same, except that the 96 bytes of packed FP6 sit in
    // 128-byte LDS rows whose last two units stay unused, so that FP6 tiles
    // copy, swizzle and read like the other 128-byte rows.
    static constexpr int ARB = Op::kARowBytes, BRB = Op::kBRowBytes;
    static constexpr int lds_units(int bytes) { return bytes == 96 ? 8 : bytes / 16; }
    static constexpr int AW = lds_units(ARB), BW = lds_units(BRB);
    static_assert(AW == 2 || AW == 4 || AW == 8, "A LDS rows of 32, 64 or 128 bytes");
    static_assert(BW == 4 || BW == 8, "B LDS rows of 64 or 128 bytes");
    static_assert((ARB != 96 && BRB != 96) || Op::kAFrag == 24, "96-byte rows hold packed FP6 only");
    static constexpr int IW = Op::kSparse ? Op::kBK / 32 : 0;                  // index words per row
    static_assert(!Op::kSparse || STEPS == 2, "index words of a k-tile read once, for two steps");
    // copy units per wave: 16-byte units of A and B, 4-byte words of the index
    static constexpr int IES = idx_copy_bytes<Op>();                           // index bytes per copy lane
    static constexpr int AUPW = BM * AW / NW, BUPW = BN * BW / NW, IUPW = BM * IW * 4 / IES / NW;
    static_assert(AUPW * NW == BM * AW && BUPW * NW == BN * BW && IUPW * NW * IES == BM * IW * 4,
                  "uneven copy split");
    static constexpr int AP = (AUPW + 63) / 64, BP = (BUPW + 63) / 64, IP = (IUPW + 63) / 64;  // passes
    // Block-scaled operands: SW scale words per row of A and per column of B
    // per k-tile, (BM + BN) * SW words in all, copied 4 bytes per lane in whole
    // passes of 64 words; pass t of wave w is the tile's pass w + t * NW.  A
    // wave left without a pass copies nothing (an offset past the buffer) into
    // a spare region of its own after the stages, so that every wave issues the
    // same number of copies and no copy sits in a branch.
    static constexpr bool SCALED = Op::kScaled;
    static constexpr int SW = Op::kScaleWords;
    static constexpr int S_WORDS = SCALED ? (BM + BN) * SW : 0, S_PASSES = S_WORDS / 64;
    static_assert(!SCALED || (BM * SW % 64 == 0 && BN * SW % 64 == 0), "whole scale copy passes");
    static constexpr int SP = SCALED ? (S_PASSES + NW - 1) / NW : 0;
    static constexpr int LPT = AP + BP + IP + SP;   // copy instructions per wave per k-tile
    static constexpr int A_BYTES = BM * AW * 16, B_BYTES = BN * BW * 16, I_BYTES = BM * IW * 4;
    static constexpr int S_BYTES = S_WORDS * 4;
    static constexpr int SPARE_BYTES = SCALED && SP * NW > S_PASSES ? NW * 256 : 0;
    static constexpr int STAGE = A_BYTES + B_BYTES + I_BYTES + S_BYTES;
    static constexpr int NSW = SCALED ? (TM + TN) * SW : 1;   // scale words a lane holds per k-tile
    // Transposed operands (A stored M-contiguous, B N-contiguous; 16- and
    // 8-bit types): the LDS tile is kBK rows of BM (BN) elements, copied row by
    // row, 16-byte unit u of row r stored at u ^ tswz(r); fragments come out of
    // it with ds_read_b64_tr_b16 (load_tr) or ds_read_b64_tr_b8 (load_tr8).
    static constexpr bool TRANS_A = TransOf<Op>::a, TRANS_B = TransOf<Op>::b;
    static_assert(!(TRANS_A || TRANS_B) || (!Op::kSparse && !SCALED), "plain dense products only");
    static constexpr int LDS_BYTES = STAGES * STAGE + SPARE_BYTES;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of a gfx950 workgroup");

    const GemmParams &p;
    int wave, lane, g, l32, wm, wn, row0, col0;
    int tm, tn, tile, split, kt0;   // output tile (row, column, number), K range, its first k-tile
    // The K walk of a whole-K tile starts at k-tile rot and wraps at nkr (see the kernel).
    int rot = 0, nkr = 0x7fffffff;
    uint8_t *spare = nullptr;   // this wave's spare LDS region (block-scaled copies)
    rsrc_t ra, rb, rx, rsa, rsb;
    acc_t acc[TM][TN];

    __device__ __forceinline__ TiledGemm(const GemmParams &p_) : p(p_) {
        const int tid = threadIdx.x;
        lane = tid & 63;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS bases go straight to M0
        g = lane >> 5;
        l32 = lane & 31;
        wm = wave / WN;
        wn = wave % WN;
        tile_coords(blockIdx.x, p, tm, tn, split);
        tile = tm * p.tiles_n + tn;
        kt0 = split * p.kt_per_split;
        row0 = tm * BM;
        col0 = tn * BN;
        const int arows = min(BM, p.M - row0), bcols = min(BN, p.N - col0);
        if constexpr (TRANS_A) ra = make_rsrc(p.A + row0 * Op::kEsize, (uint32_t)(p.K * p.a_pitch - row0 * Op::kEsize));
        else ra = make_rsrc(p.A + (int64_t)row0 * p.a_pitch, (uint32_t)(arows * p.a_pitch));
        if constexpr (TRANS_B) rb = make_rsrc(p.B + col0 * Op::kEsize, (uint32_t)(p.K * p.b_pitch - col0 * Op::kEsize));
        else rb = make_rsrc(p.B + (int64_t)col0 * p.b_pitch, (uint32_t)(bcols * p.b_pitch));
        if constexpr (Op::kSparse)
            rx = make_rsrc(p.idx + (int64_t)row0 * p.idx_pitch, (uint32_t)(arows * p.idx_pitch * 4));
        if constexpr (SCALED) {
            rsa = make_rsrc(p.sa + row0, (uint32_t)((p.scale_rows * p.ldsa - row0) * 4));
            rsb = make_rsrc(p.sb + col0, (uint32_t)((p.scale_rows * p.ldsb - col0) * 4));
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = acc_t{};
    }

    // Matrix k-tile of step kt of this workgroup's K walk.
    __device__ __forceinline__ int kabs(int kt) const {
        const int k = kt + rot;
        return (k >= nkr ? k - nkr : k) + kt0;
    }

    // Physical LDS unit P of a W-unit-wide tile -> byte offset of its source in
    // the row-major source buffer at k-tile kt.
    template <int W, int RB>
    __device__ __forceinline__ uint32_t src_off(uint32_t P, int64_t pitch, int kt) const {
        const uint32_t L = swz<W>(P);
        return (L / W) * (uint32_t)pitch + (uint32_t)(kabs(kt) * RB) + (L % W) * 16;
    }
    // Whether physical unit P of a tile of W-unit LDS rows holding RB bytes each
    // carries data (packed FP6: units 6 and 7 of a row do not).
    template <int W, int RB>
    __device__ __forceinline__ static constexpr bool data_slot(uint32_t P) {
        if constexpr (W * 16 == RB) return true;
        else return (swz<W>(P) % W) * 16 < (uint32_t)RB;
    }

    // Byte offset of the source of index copy lane d (LDS bytes [d*IES,
    // (d+1)*IES) of the row-major tile of IW words per row) at k-tile kt.
    __device__ __forceinline__ uint32_t idx_off(uint32_t d, int kt) const {
        const uint32_t byte = d * IES, r = byte / (IW * 4);
        return (r * (uint32_t)p.idx_pitch + kabs(kt) * IW) * 4 + byte % (IW * 4);
    }

    // Transposed tiles: XOR of the 16-byte unit index of row r (U units per
    // row).  16-bit elements: each ds_read_b64_tr_b16 of load_tr reads, per 32
    // lanes, 4 rows x 64 bytes; rows r .. r+3 then land in distinct quarters
    // of the 64 banks.  8-bit elements: each ds_read_b64_tr_b8 of load_tr8
    // reads, per 32 lanes, 8 rows x two adjacent units; the even XOR
    // 2 * (row number within the rows that share a 256-byte bank row) gives
    // those 16 units distinct bank groups.
    template <int U>
    __device__ __forceinline__ static constexpr uint32_t tswz(uint32_t r) {
        if constexpr (Op::kEsize == 2) return (r % 4) * (U >= 16 ? 4 : U / 4);
        else {
            static_assert(U >= 4 && U <= 16, "rows of 64 to 256 bytes");
            return 2 * ((r / (16 / U)) % (U / 2));
        }
    }
    // Source byte offset of physical unit P of a transposed tile of MN
    // elements per row at k-tile kt (memory rows are K rows of pitch bytes).
    template <int MN>
    __device__ __forceinline__ uint32_t tsrc_off(uint32_t P, int64_t pitch, int kt) const {
        constexpr int U = MN * Op::kEsize / 16;
        const uint32_t r = P / U, u = (P % U) ^ tswz<U>(r);
        return (uint32_t)(((int64_t)kabs(kt) * Op::kBK + r) * pitch) + u * 16;
    }
    template <bool T, int MN, int W, int RB>
    __device__ __forceinline__ uint32_t op_off(uint32_t P, int64_t pitch, int kt) const {
        if constexpr (T) return tsrc_off<MN>(P, pitch, kt);
        else return src_off<W, RB>(P, pitch, kt);
    }

    // Copy instruction j (0 <= j < LPT: the A passes, then B, then the index or the scales)
    // of k-tile kt into LDS stage `st`; each writes one contiguous run of LDS.
    __device__ __forceinline__ void dma_pass(uint8_t *st, int kt, int j) const {
        if (j < AP) {
            const int u = j * 64 + lane;
            if (AUPW % 64 == 0 || u < AUPW) {
                // an unused unit of a packed-FP6 row loads from past the buffer (zero, no memory
                // access) instead of branching around the copy
                const uint32_t P = wave * AUPW + u;
                const uint32_t off =
                    data_slot<AW, ARB>(P) ? op_off<TRANS_A, BM, AW, ARB>(P, p.a_pitch, kt) : kOutOfRange;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(st + (wave * AUPW + j * 64) * 16), 16, off,
                                                         0, 0, 0);
            }
        } else if (j < AP + BP) {
            const int q = j - AP, u = q * 64 + lane;
            if (BUPW % 64 == 0 || u < BUPW) {
                const uint32_t P = wave * BUPW + u;
                const uint32_t off =
                    data_slot<BW, BRB>(P) ? op_off<TRANS_B, BN, BW, BRB>(P, p.b_pitch, kt) : kOutOfRange;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(st + A_BYTES + (wave * BUPW + q * 64) * 16),
                                                         16, off, 0, 0, 0);
            }
        } else if constexpr (Op::kSparse) {
            const int q = j - AP - BP, u = q * 64 + lane;
            if (IUPW % 64 == 0 || u < IUPW)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rx, (lds_void *)(st + A_BYTES + B_BYTES + (wave * IUPW + q * 64) * IES), IES,
                    idx_off(wave * IUPW + u, kt), 0, 0, 0);
        } else if constexpr (SCALED) {
            // scale word w of the k-tile: A's words first (w = c * BM + r: word c of row r), then B's;
            // source word (kabs(kt) * SW + c) * ld + r of the operand's scale array
            const int gp = wave + (j - AP - BP) * NW;   // the tile's scale pass (wave-uniform)
            const bool real = gp < S_PASSES, on_a = gp * 64 < BM * SW;
            const int w = gp * 64 + lane - (on_a ? 0 : BM * SW);
            const int c = on_a ? w / BM : w / BN, r = on_a ? w % BM : w % BN;
            const int64_t ld = on_a ? p.ldsa : p.ldsb;
            const uint32_t off = real ? (uint32_t)((((int64_t)kabs(kt) * SW + c) * ld + r) * 4) : kOutOfRange;
            uint8_t *dst = real ? st + A_BYTES + B_BYTES + I_BYTES + gp * 256 : spare;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(on_a ? rsa : rsb, (lds_void *)dst, 4, off, 0, 0, 0);
        }
    }

    // Start the whole copy of k-tile kt into LDS stage `st` (LPT instructions per wave).
    __device__ __forceinline__ void dma(uint8_t *st, int kt) const {
#pragma unroll
        for (int j = 0; j < LPT; ++j) dma_pass(st, kt, j);
    }

    // The ragged last k-tile: A and B through registers with elements past K set
    // to zero (the index words, if any, still by copy).
    __device__ __forceinline__ void fill_masked(uint8_t *st, int kt) const {
        constexpr int EB = ElemBits<Op>::value;
        // bytes of A's (compressed) and B's rows before K, in units of kEsize
        const int climit = (Op::kSparse ? p.K / 2 : p.K) * EB / 8 / Op::kEsize;
        const int blimit = p.K * EB / 8 / Op::kEsize;
#pragma unroll
        for (int q = 0; q < AP; ++q) {
            const int u = q * 64 + lane;
            const uint32_t P = wave * AUPW + u;
            if ((AUPW % 64 == 0 || u < AUPW) && data_slot<AW, ARB>(P)) {
                if constexpr (TRANS_A) {   // whole rows of K
                    const bool in = kabs(kt) * Op::kBK + (int)(P / (BM * Op::kEsize / 16)) < p.K;
                    *reinterpret_cast<i32x4 *>(st + P * 16) =
                        in ? __builtin_amdgcn_raw_buffer_load_b128(ra, tsrc_off<BM>(P, p.a_pitch, kt), 0, 0)
                           : i32x4{0, 0, 0, 0};
                } else {
                    const int e0 = (kabs(kt) * ARB + (int)(swz<AW>(P) % AW) * 16) / Op::kEsize;
                    *reinterpret_cast<i32x4 *>(st + P * 16) =
                        masked_unit<Op::kEsize>(ra, src_off<AW, ARB>(P, p.a_pitch, kt), e0, climit);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < BP; ++q) {
            const int u = q * 64 + lane;
            const uint32_t P = wave * BUPW + u;
            if ((BUPW % 64 == 0 || u < BUPW) && data_slot<BW, BRB>(P)) {
                if constexpr (TRANS_B) {
                    const bool in = kabs(kt) * Op::kBK + (int)(P / (BN * Op::kEsize / 16)) < p.K;
                    *reinterpret_cast<i32x4 *>(st + A_BYTES + P * 16) =
                        in ? __builtin_amdgcn_raw_buffer_load_b128(rb, tsrc_off<BN>(P, p.b_pitch, kt), 0, 0)
                           : i32x4{0, 0, 0, 0};
                } else {
                    const int e0 = (kabs(kt) * BRB + (int)(swz<BW>(P) % BW) * 16) / Op::kEsize;
                    *reinterpret_cast<i32x4 *>(st + A_BYTES + P * 16) =
                        masked_unit<Op::kEsize>(rb, src_off<BW, BRB>(P, p.b_pitch, kt), e0, blimit);
                }
            }
        }
#pragma unroll
        for (int j = AP + BP; j < LPT; ++j) dma_pass(st, kt, j);   // the index words, by copy
    }

    typedef Frag<Op::kAFrag> FragA;
    typedef Frag<Op::kBFrag> FragB;
    template <class O, bool S = O::kSparse> struct IdxOf { typedef i32x2 type; };
    template <class O> struct IdxOf<O, true> { typedef typename O::idx_t type; };
    typedef typename IdxOf<Op>::type IdxT;      // index words a lane holds for one k-tile

    // Fragments of step s of the k-tile held in LDS stage `st`, and with step 0
    // the index words of every step of that k-tile (sparse A).
    __device__ __forceinline__ void load_frags(FragA (&a)[TM], FragB (&b)[TN], IdxT (&ix)[TM], uint32_t (&sw)[NSW],
                                               const uint8_t *st, int s) const {
        const uint8_t *sa = st, *sb = st + A_BYTES;
        const uint32_t *sx = reinterpret_cast<const uint32_t *>(st + A_BYTES + B_BYTES);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const uint32_t r = wm * WTM + i * 32 + l32;
            if constexpr (TRANS_A) load_tr_any<BM>(a[i], sa, wm * WTM + i * 32, s);
            else if constexpr (Op::kAFrag == 24) lds_frag6<AW>(a[i], sa, r, s);
            else lds_frag<AW>(a[i], sa, r * AW + Op::a_unit(s, g, 0), r * AW + Op::a_unit(s, g, 1));
            if constexpr (Op::kSparse) {
                if (s == 0) ix[i] = Op::load_idx(reinterpret_cast<const uint8_t *>(sx + r * IW), g);
            } else {
                ix[i] = IdxT{};
            }
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const uint32_t r = (wn * WTN + j * 32 + l32) * BW;
            if constexpr (TRANS_B) load_tr_any<BN>(b[j], sb, wn * WTN + j * 32, s);
            else if constexpr (Op::kBFrag == 24) lds_frag6<BW>(b[j], sb, wn * WTN + j * 32 + l32, s);
            else lds_frag<BW>(b[j], sb, r + Op::b_unit(s, g, 0), r + Op::b_unit(s, g, 1));
        }
        if constexpr (SCALED) {
            if (s == 0) {   // this lane's row / column scale words of the whole k-tile
                const uint32_t *ss = reinterpret_cast<const uint32_t *>(st + A_BYTES + B_BYTES + I_BYTES);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int c = 0; c < SW; ++c) sw[i * SW + c] = ss[c * BM + wm * WTM + i * 32 + l32];
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int c = 0; c < SW; ++c) sw[(TM + j) * SW + c] = ss[BM * SW + c * BN + wn * WTN + j * 32 + l32];
            }
        }
    }

    // Packed FP6 fragment: the 24 bytes of block 2s + g of row r of a tile of
    // 96 data bytes per row, bytes 48s + 24g .. + 23 of the row.  Two whole-unit reads:
    // unit 3s + 2g (lane half 0: operand bytes 0-15; half 1: bytes 8-23) and
    // unit 3s + 1, whose low half ends block 2s and whose high half starts
    // block 2s + 1; each half then puts the pieces in operand order.  (8-byte
    // reads at the blocks' own offsets would need no reordering, but every 32
    // lanes of such a read meet the same banks at least twice.)
    template <int W>
    __device__ __forceinline__ void lds_frag6(Frag<24> &f, const uint8_t *base, uint32_t r, int s) const {
        static_assert(W == 8, "96 data bytes in 128-byte LDS rows");
        f.x = *reinterpret_cast<const i32x4 *>(base + swz<W>(r * W + 3 * s + 2 * g) * 16);
        f.z = *reinterpret_cast<const i32x4 *>(base + swz<W>(r * W + 3 * s + 1) * 16);
    }

    // Fragment of the 32 rows (A) or columns (B) mn0 .. mn0 + 31 of a
    // transposed tile at step s, in the order lds_frag gives the
    // K-contiguous tiles: lane half g holds K 16s + 8g .. 16s + 8g + 7.
    // ds_read_b64_tr_b16 works on groups of 16 lanes: if lane l of a group
    // addresses 4 consecutive elements S[l][0..3], lane i receives
    // S[4e + i/4][i mod 4] for e = 0..3 (measured on gfx950).  So lane l
    // addresses row k0 + l/4, elements n0 + 4(l mod 4) .. + 3, and lane i then
    // holds rows k0 .. k0 + 3 of element n0 + i.  Group h of the wave takes
    // elements n0 = mn0 + 16(h mod 2) and K half h / 2; two reads give 8 K.
    template <int MN>
    __device__ __forceinline__ void load_tr(Frag<16> &f, const uint8_t *tile, int mn0, int s) const {
        constexpr int U = MN / 8;
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        const int h = lane >> 4, l = lane & 15;
        const int n = mn0 + 16 * (h & 1) + 4 * (l & 3);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int k = 16 * s + 8 * (h >> 1) + 4 * c + (l >> 2);
            const uint8_t *addr = tile + k * (MN * 2) + (((uint32_t)(n >> 3) ^ tswz<U>(k)) << 4) + (n & 7) * 2;
            const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)addr);
            const i32x2 w = __builtin_bit_cast(i32x2, v);
            f.v[2 * c] = w[0];
            f.v[2 * c + 1] = w[1];
        }
    }

    // The same for 8-bit elements: lane half g holds the instruction's
    // Op::kAFrag consecutive K of its row (column) in operand order, K
    // s * kKStep + g * kAFrag + 0 .. kAFrag - 1, as lds_frag gives them.
    // ds_read_b64_tr_b8 works on groups of 16 lanes: if lane l of a group
    // addresses 8 consecutive elements S[l][0..7], lane i receives
    // S[2e + i/8][i mod 8] for e = 0..7 (measured on gfx950).  So lane l
    // addresses row k0 + l/2, elements n0 + 8(l mod 2) .. + 7, and lane i then
    // holds rows k0 .. k0 + 7 of element n0 + i.  Group h of the wave takes
    // elements n0 = mn0 + 16(h mod 2) and lane half h / 2; each read gives 8 K.
    template <int MN, int BYTES>
    __device__ __forceinline__ void load_tr8(Frag<BYTES> &f, const uint8_t *tile, int mn0, int s) const {
        constexpr int U = MN / 16;
        typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
        const int h = lane >> 4, l = lane & 15;
        const int n = mn0 + 16 * (h & 1) + 8 * (l & 1);
        int w[BYTES / 4];
#pragma unroll
        for (int c = 0; c < BYTES / 8; ++c) {
            const int k = s * Op::kKStep + (h >> 1) * BYTES + 8 * c + (l >> 1);
            const uint8_t *addr = tile + k * MN + (((uint32_t)(n >> 4) ^ tswz<U>(k)) << 4) + (n & 15);
            const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)addr);
            w[2 * c] = v[0];
            w[2 * c + 1] = v[1];
        }
        if constexpr (BYTES == 16) {
            f.v = i32x4{w[0], w[1], w[2], w[3]};
        } else {
            f.lo = i32x4{w[0], w[1], w[2], w[3]};
            f.hi = i32x4{w[4], w[5], w[6], w[7]};
        }
    }
    template <int MN, int BYTES>
    __device__ __forceinline__ void load_tr_any(Frag<BYTES> &f, const uint8_t *tile, int mn0, int s) const {
        if constexpr (Op::kEsize == 2) load_tr<MN>(f, tile, mn0, s);
        else load_tr8<MN>(f, tile, mn0, s);
    }

    // Scale bytes of blocks past K (in the ragged last k-tile) become 127
    // (2^0): their elements are zero, and a 255 (NaN) there must not reach
    // the sum.  `valid` = blocks of the k-tile that lie before K.
    __device__ __forceinline__ static void mask_scales(uint32_t (&sw)[NSW], int valid) {
        if constexpr (SCALED) {
#pragma unroll
            for (int w = 0; w < NSW; ++w) {
                const int n = min(max(valid - 4 * (w % SW), 0), 4);
                const uint32_t keep = n >= 4 ? 0xffffffffu : (1u << (8 * n)) - 1u;
                sw[w] = (sw[w] & keep) | (0x7f7f7f7fu & ~keep);
            }
        }
    }

    // LDS read instructions per fragment (packed FP6: two 16-byte reads).
    static constexpr int frag_reads(int bytes) { return bytes == 24 ? 2 : bytes / 16; }
    // Instruction counts of one step, for the interleaving below.
    static constexpr int NMMA = TM * TN;
    static constexpr int NREAD = TM * frag_reads(Op::kAFrag) + TN * frag_reads(Op::kBFrag) + (Op::kSparse ? TM : 0) +
                                 (SCALED ? (TM + TN) * SW : 0);

    // Index operand of the matrix instruction of step s.
    __device__ __forceinline__ uint32_t step_idx(const IdxT &x, int s) const {
        if constexpr (Op::kSparse) return Op::lane_idx(x, s, g);
        else return 0;
    }

    // The TM x TN matrix instructions of one step, interleaved by the scheduler
    // with the LDS reads (next step's fragments) and copy instructions issued
    // before them in the same region: one matrix instruction, then one read,
    // then one copy, so the reads and copies go out while the matrix unit works.
    __device__ __forceinline__ void mma_step(const FragA (&a)[TM], const FragB (&b)[TN], const IdxT (&ix)[TM],
                                             const uint32_t (&sw)[NSW], int s, int ncopies) {
        if constexpr (SCALED) {
            // lane half g of step s holds block q = 2s + g of the k-tile (64 K per step): byte q % 4 of
            // word q / 4 of its row's and column's scale words
            const int q = 2 * s + g;
            const uint32_t sh = 8 * (q & 3);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = Op::mma_scaled(a[i], b[j], acc[i][j], sw[i * SW + (q >> 2)] >> sh,
                                               sw[(TM + j) * SW + (q >> 2)] >> sh);
        } else {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = Op::mma(a[i], b[j], acc[i][j], step_idx(ix[i], s));
        }
#pragma unroll
        for (int k = 0; k < NMMA; ++k) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            if (k < NREAD) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
            if (k < ncopies) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
        }
    }

    // Fragment double buffer: a0/b0/x0 feed the current step, a1/b1/x1 receive the next.
    FragA a0[TM], a1[TM];
    FragB b0[TN], b1[TN];
    IdxT x0[TM], x1[TM];
    uint32_t sw0[NSW], sw1[NSW];   // scale words of the current and the next k-tile

    // One k-tile: start the copy of k-tile kt + STAGES - 1 into the stage that
    // k-tile kt - 1 freed, then the STEPS steps of k-tile kt (in stage `cur`).
    // The barrier that hands over k-tile kt + 1 sits before the last step, so
    // the first fragments of k-tile kt + 1 are read while that step runs; every
    // read of a stage completes before the barrier that precedes the copy into
    // it.  STEADY: every k-tile up to kt + STAGES - 1 is whole (no branches).
    // Steady k-tiles issue their copies in two halves: P0 instructions with the
    // first step, the rest right after the barrier, with the last step, so the
    // texture-address queue sees a steadier stream than all waves issuing every
    // copy at once after the barrier.  Loads complete in issue order, so the
    // wait before the barrier may leave this k-tile's first P0 copies and the
    // STAGES - 3 whole k-tiles before them in flight.
    //
    // With two stages the stage of k-tile kt is free right after the barrier
    // of k-tile kt (its last step already holds its fragments in registers), so
    // the copy of k-tile kt + 2 goes out there, into that stage, and has STEPS
    // steps to land before the barrier of k-tile kt + 1 drains it.
    static constexpr bool TWO = STAGES == 2;
    static constexpr int AHEAD = TWO ? 2 : STAGES - 1;          // k-tile copied during k-tile kt: kt + AHEAD
    static constexpr int P0 = TWO ? 0 : LPT - LPT / 2;
    static constexpr int STEADY_WAIT = TWO ? 0 : (STAGES - 3) * LPT + P0;

    template <bool STEADY>
    __device__ __forceinline__ void iteration(uint8_t *smem, int kt, int cur, int nk, int nkt) {
        const int pre = kt + AHEAD;
        uint8_t *st_pre = smem + (TWO ? cur : (cur == 0 ? STAGES - 1 : cur - 1)) * STAGE;
        if constexpr (STEADY) {
#pragma unroll
            for (int j = 0; j < P0; ++j) dma_pass(st_pre, pre, j);
        } else if (!TWO && pre < nkt) {
            if (pre < nk) dma(st_pre, pre);
            else fill_masked(st_pre, pre);
        }
        const uint8_t *sc = smem + cur * STAGE;
        const uint8_t *sn = smem + (cur + 1 == STAGES ? 0 : cur + 1) * STAGE;
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            if (s + 1 < STEPS) {
                load_frags(a1, b1, x1, sw1, sc, s + 1);
            } else {
                if constexpr (STEADY) {
                    wait_vm_lgkm0<STEADY_WAIT>();
                } else if constexpr (TWO) {
                    wait_vm_lgkm0<0>();
                } else {
                    const int after = min(STAGES - 2, nkt - 2 - kt);
                    wait_copies<LPT, STAGES - 2>(after <= 0 || kt + 1 + after >= nk ? 0 : after);
                }
                block_barrier();
                if constexpr (STEADY) {
#pragma unroll
                    for (int j = P0; j < LPT; ++j) dma_pass(st_pre, pre, j);
                } else if (TWO && pre < nkt) {
                    if (pre < nk) dma(st_pre, pre);
                    else fill_masked(st_pre, pre);
                }
                load_frags(a1, b1, x1, sw1, sn, 0);   // past the last k-tile this reads a stale stage, unused
                if constexpr (SCALED && !STEADY)
                    if (kt + 1 == nk && nkt > nk) mask_scales(sw1, p.K / 32 - (kt0 + nk) * 4 * SW);
            }
            const int ncopies = !STEADY ? 0 : (s + 1 == STEPS ? LPT - P0 : (s == 0 ? P0 : 0));
            mma_step(a0, b0, x0, sw0, s, ncopies);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                a0[i] = a1[i];
                if (s + 1 == STEPS) x0[i] = x1[i];   // index words change once per k-tile
            }
            if constexpr (SCALED) {
                if (s + 1 == STEPS) {
#pragma unroll
                    for (int w = 0; w < NSW; ++w) sw0[w] = sw1[w];
                }
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) b0[j] = b1[j];
        }
    }

    // Split-K fix-up, after this workgroup's K range.  Every range writes its
    // partial tile (in the accumulator's register order: per instruction tile
    // and group of 4 registers, 16 bytes per thread, so each store
    // instruction covers 1 KiB) with device-scope stores, waits until they
    // have completed, and then counts itself in with one atomic add on the
    // tile's counter.  The range that arrives last resets the counter to
    // zero and sums the partials, read with device-scope loads, in range
    // order 0, 1, ..., splits - 1 (its own from registers), so the result does
    // not depend on which range finished last; it alone goes on to the
    // epilogue.  No workgroup waits for another.  Device scope on the partial
    // accesses themselves (the SC1 cache-policy bit: the data goes to and
    // comes from the memory side of the XCDs' L2 caches, which are not
    // coherent with each other) replaces whole-L2 write-back and invalidate
    // fences, which stall every workgroup of the XCD.  Returns true in the
    // last workgroup.  The arrival rank reaches the other threads through the
    // first LDS word (the k-tile stages are no longer read by then); a second
    // LDS array for it would make the compiler wait for every outstanding
    // copy before LDS reads in the main loop.
    static constexpr int SLOT_BYTES = BM * BN * 4;
    __device__ __forceinline__ bool fixup(uint32_t *arrived) {
        const int S = p.splits;
        uint8_t *tile_ws = p.partials + (int64_t)tile * S * SLOT_BYTES;
        const int tid = threadIdx.x;
        {
            const rsrc_t rw = make_rsrc(tile_ws + (int64_t)split * SLOT_BYTES, SLOT_BYTES);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int G4 = 0; G4 < 4; ++G4) {
                        // elements copied to scalars first: a bit cast of a vector
                        // element expression reads the vector's first element
                        const out_t e0 = acc[i][j][4 * G4], e1 = acc[i][j][4 * G4 + 1],
                                    e2 = acc[i][j][4 * G4 + 2], e3 = acc[i][j][4 * G4 + 3];
                        const i32x4 v = {__builtin_bit_cast(int, e0), __builtin_bit_cast(int, e1),
                                         __builtin_bit_cast(int, e2), __builtin_bit_cast(int, e3)};
                        const uint32_t o = (uint32_t)((((i * TN + j) * 4 + G4) * NT + tid) * 16);
                        __builtin_amdgcn_raw_buffer_store_b128(v, rw, o, 0, kDeviceScope);
                    }
        }
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this thread's partial has reached device scope
        __syncthreads();
        if (tid == 0) {
            const uint32_t before = __hip_atomic_fetch_add(p.counters + tile, 1u, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
            if (before == (uint32_t)S - 1)
                __hip_atomic_store(p.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *arrived = before;
        }
        __syncthreads();
        const bool last = *arrived == (uint32_t)S - 1;
        __syncthreads();   // read by every wave before the epilogue reuses the LDS
        if (!last) return false;
        // acc = p_0 + p_1 + ... in range order
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int G4 = 0; G4 < 4; ++G4) {
                    const uint32_t o = (uint32_t)((((i * TN + j) * 4 + G4) * NT + tid) * 16);
                    out_t sum[4];
                    for (int s = 0; s < S; ++s) {
                        out_t x[4];
                        if (s == split) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) x[e] = acc[i][j][4 * G4 + e];
                        } else {
                            const rsrc_t rr = make_rsrc(tile_ws + (int64_t)s * SLOT_BYTES, SLOT_BYTES);
                            const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rr, o, 0, kDeviceScope);
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const int w = v[e];
                                x[e] = __builtin_bit_cast(out_t, w);
                            }
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (s == 0) sum[e] = x[e];
                            else if constexpr (std::is_same<out_t, float>::value) sum[e] = sum[e] + x[e];
                            else sum[e] = (int32_t)((uint32_t)sum[e] + (uint32_t)x[e]);
                        }
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][j][4 * G4 + e] = sum[e];
                }
        return true;
    }

    // D = alpha * acc + beta * C, then (floating inputs) the column bias, ReLU
    // and rounding to D's type.  Element (i, j) of a 32 x 32 instruction tile
    // is register G of lane L with i = 8*floor(G/4) + 4*floor(L/32) + (G mod 4),
    // j = L mod 32, so for each register lanes 0-31 and 32-63 each cover 32
    // consecutive elements of a row.  C and D are accessed with buffer
    // instructions over this tile's rows: elements outside M x N get an offset
    // past the end of the buffer, where loads return zero and stores are
    // dropped, so there are no branches and all loads of a row of instruction
    // tiles are in flight together.  fp32 / int32 D takes the unrolled paths
    // below; 16- and 8-bit D the converted path after them.
    __device__ __forceinline__ void epilogue(uint8_t *smem) {
        if constexpr (std::is_same<out_t, float>::value) {
            if (p.d_type != OUT_ACC) return epilogue_converted(smem);
        }
        const int rows = min(BM, p.M - row0);
        const rsrc_t rd = make_rsrc(reinterpret_cast<out_t *>(p.D) + (int64_t)row0 * p.ldd,
                                    (uint32_t)(rows * p.ldd * 4));
        float bias[TN];   // this lane's column of each instruction-tile column
        const bool has_bias = load_bias(bias);
        if (p.use_c && !p.fold_c) {
            const rsrc_t rc = make_rsrc(reinterpret_cast<const out_t *>(p.C) + (int64_t)row0 * p.ldc,
                                        (uint32_t)(rows * p.ldc * 4));
            store_tiles<true>(rd, rc, bias, has_bias);
        } else if (p.vec_d) {
            store_tiles_lds(rd, smem, bias, has_bias);
        } else {
            store_tiles<false>(rd, rd, bias, has_bias);
        }
    }

    // The bias of this lane's column of each instruction-tile column (floating
    // D only); returns whether there is a bias.
    __device__ __forceinline__ bool load_bias(float (&bias)[TN]) const {
        const bool has_bias = std::is_same<out_t, float>::value && p.bias != nullptr;
#pragma unroll
        for (int j = 0; j < TN; ++j) bias[j] = 0.0f;
        if (has_bias) {
            const rsrc_t rb = make_rsrc(p.bias + col0, (uint32_t)(min(BN, p.N - col0) * 4));
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int c = wn * WTN + j * 32 + l32;   // column within the block tile
                bias[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                        rb, col0 + c < p.N ? (uint32_t)c * 4 : kOutOfRange, 0, 0));
            }
        }
        return has_bias;
    }

    // One fp32 / int32 output element's bits from its accumulator value and
    // (USE_C) the bits of its C element.
    template <bool USE_C, class A>
    __device__ __forceinline__ uint32_t out_bits(A a, uint32_t c, float bias, bool has_bias) const {
        if constexpr (std::is_same<out_t, float>::value) {
            float v = p.alpha * a;
            if constexpr (USE_C) v = fmaf(p.beta, __builtin_bit_cast(float, c), v);
            return finish<OUT_ACC>(v, bias, has_bias, p.act != 0);
        } else {
            uint32_t v = (uint32_t)p.ialpha * (uint32_t)a;
            if constexpr (USE_C) v += (uint32_t)p.ibeta * c;
            return v;
        }
    }

    // The epilogue through LDS (free once the last k-tile is done: no copy is
    // in flight and no remaining read matters), so that D goes out with
    // 16-byte stores, each instruction writing 8 whole 128-byte row segments
    // instead of 2.  Each wave stages up to EPI_TILES of its 32 x 32 instruction
    // tiles at a time in its own 4 KiB-per-tile region (no other wave touches
    // it, so no barrier): lanes write their 16 registers in the accumulator
    // layout, then read back row-contiguous 16-byte chunks (lane L: row
    // 8q + L / 8 of the tile, chunk L mod 8).  Row r of a tile sits at row
    // slot r ^ ((r >> 2) & 1): rows r and r + 4, written by the two lane halves
    // together, then fall in opposite halves of the 64 banks, and so do the two
    // rows of each 16-lane read.
    static constexpr int epi_tiles() {   // most instruction tiles per pass: fits and divides TM * TN
        int t = TM * TN;
        while (t > 1 && (t * 4096 * NW > STAGES * STAGE || (TM * TN) % t != 0)) --t;
        return t;
    }
    static constexpr int EPI_TILES = epi_tiles();
    static_assert(EPI_TILES * 4096 * NW <= STAGES * STAGE, "epilogue staging space (the stages, not the spare)");

    // Stage t of the current group: this lane's 16 values of instruction tile (i, j), as fp32 / int32 bits.
    template <class F>
    __device__ __forceinline__ void stage_tile(uint8_t *base, int i, int j, F bits_of) {
#pragma unroll
        for (int G = 0; G < 16; ++G) {
            const int r = 8 * (G / 4) + 4 * g + (G % 4);
            const int slot = r ^ ((r >> 2) & 1);
            *reinterpret_cast<uint32_t *>(base + slot * 128 + l32 * 4) = bits_of(acc[i][j][G]);
        }
    }

    __device__ __forceinline__ void store_tiles_lds(rsrc_t rd, uint8_t *smem, const float *bias, bool has_bias) {
        uint8_t *region = smem + wave * EPI_TILES * 4096;
#pragma unroll
        for (int t0 = 0; t0 < TM * TN; t0 += EPI_TILES) {
#pragma unroll
            for (int t = 0; t < EPI_TILES; ++t) {
                const int i = (t0 + t) / TN, j = (t0 + t) % TN;
                stage_tile(region + t * 4096, i, j,
                           [&](out_t a) { return out_bits<false>(a, 0u, bias[j], has_bias); });
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's staging writes are done
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < EPI_TILES; ++t) {
                const int i = (t0 + t) / TN, j = (t0 + t) % TN;
                const uint8_t *base = region + t * 4096;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = 8 * q + lane / 8, c = lane % 8;
                    const int slot = r ^ ((r >> 2) & 1);
                    const i32x4 v = *reinterpret_cast<const i32x4 *>(base + slot * 128 + c * 16);
                    const int tr = wm * WTM + i * 32 + r;                    // row within the block tile
                    const int col = col0 + wn * WTN + j * 32 + 4 * c;       // first of the 4 columns
                    const bool rin = row0 + tr < p.M;
                    const uint32_t o = (uint32_t)((tr * p.ldd + col) * 4);
                    if (col + 3 < p.N) {
                        __builtin_amdgcn_raw_buffer_store_b128(v, rd, rin ? o : kOutOfRange, 0, kNonTemporal);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            __builtin_amdgcn_raw_buffer_store_b32((uint32_t)v[e], rd,
                                                                  rin && col + e < p.N ? o + 4 * e : kOutOfRange, 0,
                                                                  kNonTemporal);
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);   // the reads are done before the region is written again
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // 16- and 8-bit C and D (floating inputs).  alpha * acc (plus the column
    // bias, when given) is staged in LDS as fp32 in the layout above; then
    // each lane reads back four consecutive columns of a row at a time and
    // finishes them there: beta * C (C has D's type and is read here, four
    // elements per load), ReLU and the rounding, in a loop unrolled only four
    // times (one short body per output type, four C loads in flight).  Four outputs leave in one
    // 8-byte (16-bit D) or 4-byte (8-bit D) store when D's rows allow (vec_d),
    // else one by one.
    __device__ __forceinline__ void epilogue_converted(uint8_t *smem) {
        if constexpr (std::is_same<out_t, float>::value) {
            switch (p.d_type) {   // one copy of the loops per output type
            case OUT_BF16: return converted_as<OUT_BF16>(smem);
            case OUT_F16: return converted_as<OUT_F16>(smem);
            case OUT_E4M3: return converted_as<OUT_E4M3>(smem);
            default: return converted_as<OUT_E5M2>(smem);
            }
        }
    }

    template <int OT>
    __device__ __forceinline__ void converted_as(uint8_t *smem) {
        constexpr int es = out_esize<OT>();
        const int rows = min(BM, p.M - row0);
        const rsrc_t rd = make_rsrc(static_cast<uint8_t *>(p.D) + (int64_t)row0 * p.ldd * es,
                                    (uint32_t)(rows * p.ldd * es));
        const rsrc_t rc = p.use_c ? make_rsrc(static_cast<const uint8_t *>(p.C) + (int64_t)row0 * p.ldc * es,
                                              (uint32_t)(rows * p.ldc * es))
                                  : rd;
        const bool relu = p.act != 0;
        float bias[TN];
        const bool has_bias = load_bias(bias);
        uint8_t *region = smem + wave * EPI_TILES * 4096;
#pragma unroll
        for (int t0 = 0; t0 < TM * TN; t0 += EPI_TILES) {
#pragma unroll
            for (int t = 0; t < EPI_TILES; ++t) {
                const int j = (t0 + t) % TN;
                stage_tile(region + t * 4096, (t0 + t) / TN, j, [&](float a) {
                    const float v = p.alpha * a;
                    return __builtin_bit_cast(uint32_t, has_bias ? v + bias[j] : v);
                });
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the staging writes are done
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll 4
            for (int k = 0; k < EPI_TILES * 4; ++k) {
                const int t = k >> 2, q = k & 3, tt = t0 + t, i = tt / TN, j = tt % TN;
                const int r = 8 * q + lane / 8, c = lane % 8;
                const int slot = r ^ ((r >> 2) & 1);
                const f32x4 v = *reinterpret_cast<const f32x4 *>(region + t * 4096 + slot * 128 + c * 16);
                const int tr = wm * WTM + i * 32 + r;                   // row within the block tile
                const int cc = wn * WTN + j * 32 + 4 * c;              // first column within the block tile
                if (row0 + tr >= p.M || col0 + cc >= p.N) continue;
                const bool whole = col0 + cc + 3 < p.N;
                const uint32_t od = (uint32_t)((tr * p.ldd + col0 + cc) * es);
                float x[4] = {v[0], v[1], v[2], v[3]};
                if (p.use_c) {
                    const uint32_t oc = (uint32_t)((tr * p.ldc + col0 + cc) * es);
                    uint32_t cb[4];
                    if (whole && p.vec_c) {
                        if constexpr (es == 2) {
                            const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(rc, oc, 0, kNonTemporal);
                            cb[0] = w[0] & 0xffffu; cb[1] = w[0] >> 16;
                            cb[2] = w[1] & 0xffffu; cb[3] = w[1] >> 16;
                        } else {
                            const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(rc, oc, 0, kNonTemporal);
                            for (int e = 0; e < 4; ++e) cb[e] = (w >> (8 * e)) & 0xffu;
                        }
                    } else {
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t oe = col0 + cc + e < p.N ? oc + es * e : kOutOfRange;
                            if constexpr (es == 2) cb[e] = __builtin_amdgcn_raw_buffer_load_b16(rc, oe, 0, kNonTemporal);
                            else cb[e] = __builtin_amdgcn_raw_buffer_load_b8(rc, oe, 0, kNonTemporal);
                        }
                    }
                    for (int e = 0; e < 4; ++e) x[e] = fmaf(p.beta, from_out_bits<OT>(cb[e]), x[e]);
                }
                uint32_t h[4];
                for (int e = 0; e < 4; ++e) h[e] = finish<OT>(x[e], 0.0f, false, relu);
                if (whole && p.vec_d) {
                    if constexpr (es == 2) {
                        const u32x2 w = {h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
                        __builtin_amdgcn_raw_buffer_store_b64(w, rd, od, 0, kNonTemporal);
                    } else {
                        __builtin_amdgcn_raw_buffer_store_b32(h[0] | (h[1] << 8) | (h[2] << 16) | (h[3] << 24), rd, od,
                                                              0, kNonTemporal);
                    }
                } else {
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t oe = col0 + cc + e < p.N ? od + es * e : kOutOfRange;
                        if constexpr (es == 2) __builtin_amdgcn_raw_buffer_store_b16((unsigned short)h[e], rd, oe, 0, kNonTemporal);
                        else __builtin_amdgcn_raw_buffer_store_b8((unsigned char)h[e], rd, oe, 0, kNonTemporal);
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);   // the reads are done before the region is written again
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Folded beta * C (fp32 / int32 D): the accumulator starts as c_scale * C,
    // read with the same branch-free buffer accesses as the epilogue.  Called
    // right after the first copies are issued, so the two latencies overlap.
    __device__ __forceinline__ void load_c_into_acc() {
        const int rows = min(BM, p.M - row0);
        const rsrc_t rc = make_rsrc(reinterpret_cast<const out_t *>(p.C) + (int64_t)row0 * p.ldc,
                                    (uint32_t)(rows * p.ldc * 4));
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int col = col0 + wn * WTN + j * 32 + l32;
#pragma unroll
                for (int G = 0; G < 16; ++G) {
                    const int r = wm * WTM + i * 32 + 8 * (G / 4) + 4 * g + (G % 4);
                    const bool in = (row0 + r < p.M) && (col < p.N);
                    const uint32_t oc = in ? (uint32_t)((r * p.ldc + col) * 4) : kOutOfRange;
                    const uint32_t c = __builtin_amdgcn_raw_buffer_load_b32(rc, oc, 0, kNonTemporal);
                    if constexpr (std::is_same<out_t, float>::value)
                        acc[i][j][G] = p.c_scale * __builtin_bit_cast(float, c);
                    else
                        acc[i][j][G] = (int32_t)((uint32_t)p.ibeta * c);
                }
            }
            __builtin_amdgcn_sched_barrier(0);   // at most one row of instruction tiles of C in flight
        }
    }

    template <bool USE_C>
    __device__ __forceinline__ void store_tiles(rsrc_t rd, rsrc_t rc, const float *bias, bool has_bias) {
        constexpr int JB = TN < 2 ? TN : 2;             // instruction tiles per batch of loads
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j0 = 0; j0 < TN; j0 += JB) {
                uint32_t c[JB][16];
                uint32_t od[JB][16];
#pragma unroll
                for (int jj = 0; jj < JB; ++jj) {
                    const int col = col0 + wn * WTN + (j0 + jj) * 32 + l32;
#pragma unroll
                    for (int G = 0; G < 16; ++G) {
                        const int r = wm * WTM + i * 32 + 8 * (G / 4) + 4 * g + (G % 4);   // row within the tile
                        const bool in = (row0 + r < p.M) && (col < p.N);
                        od[jj][G] = in ? (uint32_t)((r * p.ldd + col) * 4) : kOutOfRange;
                        c[jj][G] = 0;
                        if constexpr (USE_C) {
                            const uint32_t oc = in ? (uint32_t)((r * p.ldc + col) * 4) : kOutOfRange;
                            c[jj][G] = __builtin_amdgcn_raw_buffer_load_b32(rc, oc, 0, kNonTemporal);
                        }
                    }
                }
#pragma unroll
                for (int jj = 0; jj < JB; ++jj) {
#pragma unroll
                    for (int G = 0; G < 16; ++G)
                        __builtin_amdgcn_raw_buffer_store_b32(
                            out_bits<USE_C>(acc[i][j0 + jj][G], c[jj][G], bias[j0 + jj], has_bias), rd, od[jj][G], 0,
                            kNonTemporal);
                }
            }
        }
    }
};

// One workgroup per CU: with WM*WN/4 waves on each SIMD every wave may use
// 512 / (WM*WN/4) registers.
template <class Op, int BM, int BN, int WM, int WN, int STAGES>
__global__ __launch_bounds__(WM *WN * 64) __attribute__((amdgpu_waves_per_eu(WM * WN / 4, WM * WN / 4)))
void gemm_tiled_kernel(GemmParams p) {
    typedef TiledGemm<Op, BM, BN, WM, WN, STAGES> T;
    __shared__ __attribute__((aligned(16))) uint8_t smem[T::LDS_BYTES];
    T t(p);
    if constexpr (T::SPARE_BYTES > 0) t.spare = smem + T::STAGES * T::STAGE + t.wave * 256;

    // this workgroup's K range: k-tiles [kt0, kt0 + nkt) of the matrix, the
    // first nk of them whole (a ragged k-tile can only be the matrix's last)
    const int nk_all = p.K / Op::kBK;
    const int nkt_all = nk_all + (p.K > nk_all * Op::kBK ? 1 : 0);
    const int kt_end = min(t.kt0 + p.kt_per_split, nkt_all);
    const int nkt = kt_end - t.kt0;
    const int nk = min(kt_end, nk_all) - t.kt0;
    // A whole-K tile (no split, no ragged k-tile) starts its K walk at k-tile (tile row + tile
    // column) mod 4 and wraps around.  Of the tiles an XCD runs at once (eight tile rows by four
    // tile columns), those sharing a k-slice of A or of B then fetch it at different times, the later
    // ones from that XCD's L2 rather than all of them together from the fabric.  Measured at 8192^3:
    // bf16 1 %, fp8 x bf8 3-4 % and 4:2 fp8 4-5 % faster.  A tile's order depends only on its
    // coordinates, so results stay deterministic, and exact sums are unchanged.
    if (p.splits == 1 && nkt == nk && nk >= 4) {
        t.rot = (t.tm + t.tn) & 3;
        t.nkr = nk;
    }

    // prologue: start k-tiles 0 .. AHEAD-1 (and the folded C, whose loads overlap them)
#pragma unroll
    for (int s = 0; s < T::AHEAD; ++s) {
        if (s < nkt) {
            if (s < nk) t.dma(smem + s * T::STAGE, s);
            else t.fill_masked(smem + s * T::STAGE, s);
        }
    }
    if (p.fold_c && t.split == 0) t.load_c_into_acc();
    // Copies are counted per wave in issue order.  Before using k-tile kt + 1 the
    // copies of the later k-tiles may stay in flight, provided they are all
    // whole k-tiles (the ragged one issues fewer copy instructions); otherwise
    // wait for everything.
    {
        const int after = min(T::AHEAD - 1, nkt - 1);
        wait_copies<T::LPT, T::AHEAD - 1>(after <= 0 || after >= nk ? 0 : after);
        block_barrier();
    }
    if (nkt > 0) t.load_frags(t.a0, t.b0, t.x0, t.sw0, smem, 0);
    if constexpr (T::SCALED)
        if (nk == 0 && nkt > 0) t.mask_scales(t.sw0, p.K / 32 - t.kt0 * 4 * T::SW);
    int kt = 0, cur = 0;
    for (; kt + T::AHEAD < nk; ++kt) {
        t.template iteration<true>(smem, kt, cur, nk, nkt);
        cur = (cur + 1 == STAGES) ? 0 : cur + 1;
    }
    for (; kt < nkt; ++kt) {
        t.template iteration<false>(smem, kt, cur, nk, nkt);
        cur = (cur + 1 == STAGES) ? 0 : cur + 1;
    }
    if (p.splits > 1 && !t.fixup(reinterpret_cast<uint32_t *>(smem))) return;
    t.epilogue(smem);
}

}  // namespace mmac
