// Skinny dense GEMM (M <= 32): D = alpha * A*B + beta * C streaming B once.
//
// With at most 32 rows of A the product does 2*M flops per byte of B, far
// below the chip's flop/byte ridge, so the time is set by reading B from HBM.
// Each workgroup owns 16*CB columns of D and all M rows; its WK waves split K
// (a fixed, contiguous range each), copy their rows of B (read exactly once)
// and A (from L2) into LDS a whole cache line at a time, run 16 x 16 matrix
// instructions on fragments read back from LDS, and combine their partial
// tiles in LDS in a fixed wave order, so the result does not depend on timing.
//
// The 16 x 16 accumulator follows the one-block 16x16 layout of "CDNA dense
// MFMA builtins", "Accumulator layout": element (i, j) is register i mod 4 of
// lane 16*floor(i/4) + j.  Within an instruction's K step, lane quarter
// q = lane / 16 takes the q-th quarter of the step for A and B alike.
#include "device.h"
#include "launch.h"

namespace mmac {

// 16 x 16 dense instructions of gfx950, one per element type.
template <int DT_A, int DT_B> struct Mma16;
template <int DT> struct Mma16Half {
    static constexpr int kEsize = 2, kFrag = 16, kKStep = 32;   // 8 elements per lane
    typedef i32x4 frag_t;
    typedef f32x4 acc_t;
    typedef float out_t;
    __device__ __forceinline__ static acc_t mma(const i32x4 &a, const i32x4 &b, acc_t c) {
        if constexpr (DT == DT_BF16)
            return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                          c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                         c, 0, 0, 0);
    }
};
template <> struct Mma16<DT_BF16, DT_BF16> : Mma16Half<DT_BF16> {};
template <> struct Mma16<DT_F16, DT_F16> : Mma16Half<DT_F16> {};
template <> struct Mma16<DT_I8, DT_I8> {
    static constexpr int kEsize = 1, kFrag = 16, kKStep = 64;    // 16 elements per lane
    typedef i32x4 frag_t;
    typedef i32x4 acc_t;
    typedef int32_t out_t;
    __device__ __forceinline__ static acc_t mma(const i32x4 &a, const i32x4 &b, acc_t c) {
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
    }
};
template <int FA, int FB> struct Mma16F8 {
    static constexpr int kEsize = 1, kFrag = 32, kKStep = 128;   // 32 elements per lane
    typedef Frag<32> frag_t;
    typedef f32x4 acc_t;
    typedef float out_t;
    __device__ __forceinline__ static acc_t mma(const Frag<32> &a, const Frag<32> &b, acc_t c) {
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(join(a), join(b), c, FA, FB, 0, 0, 0, 0);
    }
};
template <> struct Mma16<DT_E4M3, DT_E4M3> : Mma16F8<0, 0> {};
template <> struct Mma16<DT_E4M3, DT_E5M2> : Mma16F8<0, 1> {};
template <> struct Mma16<DT_E5M2, DT_E4M3> : Mma16F8<1, 0> {};
template <> struct Mma16<DT_E5M2, DT_E5M2> : Mma16F8<1, 1> {};

// 16 bytes of a row at byte offset `off`, elements at or past `limit` (element
// index e0 is the first) read as zero.
template <int ES>
__device__ __forceinline__ i32x4 load_unit(rsrc_t r, uint32_t off, int e0, int limit) {
    constexpr int PER = 16 / ES;
    if (e0 + PER <= limit) return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    uint32_t w[4] = {0, 0, 0, 0};
    for (int e = 0; e < PER; ++e) {
        if (e0 + e < limit) {
            uint32_t x;
            if constexpr (ES == 2) x = __builtin_amdgcn_raw_buffer_load_b16(r, off + 2 * e, 0, 0);
            else x = __builtin_amdgcn_raw_buffer_load_b8(r, off + e, 0, 0);
            w[(e * ES) / 4] |= x << (8 * ((e * ES) % 4));
        }
    }
    return i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
}

// The fragment of one K step (starting at element k0) of the row at row_off,
// straight into registers, elements past K zero: the masked path for the
// chunk that K ends inside.
template <class Op>
__device__ __forceinline__ void load_frag16(typename Op::frag_t &f, rsrc_t r, uint32_t row_off, int k0, int K,
                                            int q) {
    constexpr int ES = Op::kEsize;
    if constexpr (Op::kFrag == 16) {
        const int e0 = k0 + q * (16 / ES);
        f = load_unit<ES>(r, row_off + (uint32_t)e0 * ES, e0, K);
    } else {
        const int e0 = k0 + q * 32;
        f.lo = load_unit<ES>(r, row_off + (uint32_t)e0, e0, K);
        f.hi = load_unit<ES>(r, row_off + (uint32_t)e0 + 16, e0 + 16, K);
    }
}

// s_waitcnt on gfx9: vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt
// [11:8].  Waits until at most VM vector-memory instructions of this wave are
// outstanding and every LDS access has completed.
template <int VM>
__device__ __forceinline__ void skinny_wait() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));
    asm volatile("" ::: "memory");
}
// The same with the count n (0 <= n <= MAXN, in units of PER instructions) known only at run time.
template <int PER, int MAXN>
__device__ __forceinline__ void skinny_wait_n(int n) {
    if constexpr (MAXN <= 0) {
        skinny_wait<0>();
    } else {
        if (n >= MAXN) skinny_wait<MAXN * PER>();
        else skinny_wait_n<PER, MAXN - 1>(n);
    }
}

// Every LDS access of this wave has completed (outstanding memory loads may remain).
__device__ __forceinline__ void skinny_wait_lds() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
    asm volatile("" ::: "memory");
}

// 16-byte unit u of row r of a 16-row block sits at unit u ^ ((r / 2) mod 8) of
// its 128-byte LDS row: the 16 lanes that read one unit of all 16 rows then
// meet 16 different 16-byte bank groups.
__device__ __forceinline__ int skinny_swz(int r) { return (r >> 1) & 7; }

// MB row blocks of 16 (M <= 16*MB), CB column blocks of 16 per workgroup, WK
// waves along K, NSLOT chunks of loads in flight per wave.
//
// The rows of A and B are read in chunks of 128 bytes, one cache line per row
// (64 16-bit or 128 8-bit elements: two instruction steps, or one for fp8).
// A copy instruction moves 8 rows x 128 bytes straight into LDS (lane l: row
// l/8, unit l mod 8), so every line is requested once.  Loaded into registers
// in the instructions' own fragment layout (16 rows x 4 lanes of 16 bytes)
// each line would be requested twice, half of it each time, and that request
// rate, not HBM, would set the time.  Each wave streams its own contiguous
// range of whole chunks through a private ring of NSLOT LDS slots and reads its
// fragments back from there (no barrier: a wave reads only what it copied); the
// chunk that K ends inside goes through registers, with the elements past K
// set to zero.  Lane (r, q) = (lane mod 16, lane / 16) takes unit 4v + q of a
// chunk in step v (16-byte fragments) or units 2q, 2q+1 (fp8's 32-byte ones):
// the K order of the plain register loads.
template <class Op, int MB, int CB, int WK, int NSLOT>
__global__ __launch_bounds__(WK * 64) void gemm_skinny_kernel(GemmParams p) {
    typedef typename Op::acc_t acc_t;
    typedef typename Op::out_t out_t;
    typedef typename Op::frag_t frag_t;
    constexpr int KS = Op::kKStep, ES = Op::kEsize;
    constexpr int CE = 128 / ES;                  // K elements per chunk
    constexpr int SPC = CE / KS;                  // instruction steps per chunk
    constexpr int BLOCKS = MB + CB;               // 16-row blocks per chunk: B's first, then A's
    constexpr int IPC = 2 * BLOCKS;               // copy instructions per chunk (8 rows each)
    constexpr int SLOT = BLOCKS * 16 * 128;       // bytes of one chunk in LDS
    constexpr int RED = WK * MB * CB * 4 * 64 * 4;
    constexpr int LDS_BYTES = WK * NSLOT * SLOT > RED ? WK * NSLOT * SLOT : RED;
    static_assert(SPC >= 1 && SPC * KS == CE, "whole steps per chunk");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, r16 = lane & 15, q = lane >> 4;
    const int col0 = blockIdx.x * 16 * CB;
    const int bcols = min(16 * CB, p.N - col0);
    const rsrc_t ra = make_rsrc(p.A, (uint32_t)(p.M * p.a_pitch));
    const rsrc_t rb = make_rsrc(p.B + (int64_t)col0 * p.b_pitch, (uint32_t)(bcols * p.b_pitch));

    // The output this thread writes after the reduction; its C element is
    // loaded now so that the load overlaps the streaming of B.  Buffer accesses
    // over D's / C's first M rows: elements outside M x N get an offset past the
    // end, where loads return zero and stores are dropped.
    constexpr int OUTS = MB * CB * 4 * 64;
    static_assert(OUTS <= WK * 64, "one output per thread");
    const int o = threadIdx.x;
    const int oln = o & 63, orr = (o >> 6) & 3, oc = (o >> 8) % CB, om = (o >> 8) / CB;
    const int orow = om * 16 + 4 * (oln >> 4) + orr, ocol = col0 + oc * 16 + (oln & 15);
    const bool oin = o < OUTS && orow < p.M && ocol < p.N;
    constexpr bool kFloat = std::is_same<out_t, float>::value;
    const int es = !kFloat || p.d_type == OUT_ACC ? 4 : p.d_type <= OUT_F16 ? 2 : 1;   // bytes of a C / D element
    const rsrc_t rd = make_rsrc(p.D, (uint32_t)(p.M * p.ldd * es));
    const uint32_t od = oin ? (uint32_t)((orow * p.ldd + ocol) * es) : kOutOfRange;
    uint32_t cpre = 0;
    if (p.use_c) {
        const rsrc_t rcc = make_rsrc(p.C, (uint32_t)(p.M * p.ldc * es));
        const uint32_t oc = oin ? (uint32_t)((orow * p.ldc + ocol) * es) : kOutOfRange;
        cpre = es == 4   ? __builtin_amdgcn_raw_buffer_load_b32(rcc, oc, 0, 0)
               : es == 2 ? __builtin_amdgcn_raw_buffer_load_b16(rcc, oc, 0, 0)
                         : __builtin_amdgcn_raw_buffer_load_b8(rcc, oc, 0, 0);
    }
    const bool has_bias = kFloat && p.bias != nullptr;
    float bias = 0.0f;
    if (has_bias)
        bias = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             make_rsrc(p.bias + col0, (uint32_t)(bcols * 4)),
                                             oin ? (uint32_t)(ocol - col0) * 4 : kOutOfRange, 0, 0));

    acc_t acc[MB][CB];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int c = 0; c < CB; ++c) acc[m][c] = acc_t{};

    // whole chunks: a contiguous range per wave
    const int nfull = p.K / CE;
    const int per = (nfull + WK - 1) / WK;
    const int c0 = min(wave * per, nfull), c1 = min(c0 + per, nfull);
    uint8_t *ring = smem + wave * NSLOT * SLOT;

    // copy instruction j of chunk c into slot `slot`: block j / 2 (B's blocks, then A's),
    // rows 8 (j mod 2) .. + 7 of it; rows past M or N read as zero (offsets past the buffer)
    auto issue = [&](int c, int slot) {
        const int r = lane >> 3;
#pragma unroll
        for (int j = 0; j < IPC; ++j) {
            const int blk = j >> 1, row = 8 * (j & 1) + r;
            const uint32_t unit = (uint32_t)((lane & 7) ^ skinny_swz(row));
            const uint32_t kb = (uint32_t)c * 128u + unit * 16u;
            uint8_t *dst = ring + slot * SLOT + j * 1024;
            if (blk < CB)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rb, (lds_void *)dst, 16, (uint32_t)(blk * 16 + row) * (uint32_t)p.b_pitch + kb, 0, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    ra, (lds_void *)dst, 16, (uint32_t)((blk - CB) * 16 + row) * (uint32_t)p.a_pitch + kb, 0, 0,
                    0);
        }
    };
    // unit u of row r16 of block blk in slot `slot`
    auto unit_at = [&](int slot, int blk, int u) -> i32x4 {
        return *reinterpret_cast<const i32x4 *>(ring + slot * SLOT + blk * 2048 + r16 * 128 +
                                               ((u ^ skinny_swz(r16)) << 4));
    };

#pragma unroll
    for (int i = 0; i < NSLOT; ++i)
        if (c0 + i < c1) issue(c0 + i, i);
    for (int c = c0; c < c1; ++c) {
        const int slot = (c - c0) % NSLOT;
        // chunk c has landed once at most the chunks issued after it are outstanding
        skinny_wait_n<IPC, NSLOT - 1>(min(NSLOT - 1, c1 - 1 - c));
        frag_t a[SPC][MB], b[SPC][CB];
#pragma unroll
        for (int v = 0; v < SPC; ++v) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                if constexpr (Op::kFrag == 16) b[v][cb] = unit_at(slot, cb, 4 * v + q);
                else { b[v][cb].lo = unit_at(slot, cb, 2 * q); b[v][cb].hi = unit_at(slot, cb, 2 * q + 1); }
            }
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                if constexpr (Op::kFrag == 16) a[v][m] = unit_at(slot, CB + m, 4 * v + q);
                else { a[v][m].lo = unit_at(slot, CB + m, 2 * q); a[v][m].hi = unit_at(slot, CB + m, 2 * q + 1); }
            }
        }
        skinny_wait_lds();   // the slot's reads are done before new data is copied into it
        if (c + NSLOT < c1) issue(c + NSLOT, slot);
#pragma unroll
        for (int v = 0; v < SPC; ++v)
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) acc[m][cb] = Op::mma(a[v][m], b[v][cb], acc[m][cb]);
    }

    // the chunk K ends inside (if any): the last wave, through registers, elements past K zero
    if (wave == WK - 1 && nfull * CE < p.K) {
        uint32_t aoff[MB], boff[CB];
#pragma unroll
        for (int m = 0; m < MB; ++m) aoff[m] = (uint32_t)(m * 16 + r16) * (uint32_t)p.a_pitch;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) boff[cb] = (uint32_t)(cb * 16 + r16) * (uint32_t)p.b_pitch;
#pragma unroll
        for (int v = 0; v < SPC; ++v) {
            const int k0 = nfull * CE + v * KS;
            if (k0 < p.K) {
                frag_t a[MB], b[CB];
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) load_frag16<Op>(b[cb], rb, boff[cb], k0, p.K, q);
#pragma unroll
                for (int m = 0; m < MB; ++m) load_frag16<Op>(a[m], ra, aoff[m], k0, p.K, q);
#pragma unroll
                for (int m = 0; m < MB; ++m)
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) acc[m][cb] = Op::mma(a[m], b[cb], acc[m][cb]);
            }
        }
    }

    // combine the WK partial tiles in LDS, in wave order; each thread then owns one output
    // (in the LDS of the chunk rings, once every wave is done with its ring)
    __syncthreads();
    out_t(*red)[MB][CB][4][64] = reinterpret_cast<out_t(*)[MB][CB][4][64]>(smem);
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int c = 0; c < CB; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][m][c][r][lane] = acc[m][c][r];
    __syncthreads();
    if (o < OUTS) {
        out_t v = red[0][om][oc][orr][oln];
        for (int w = 1; w < WK; ++w) {
            if constexpr (std::is_same<out_t, float>::value) v += red[w][om][oc][orr][oln];
            else v = (out_t)((uint32_t)v + (uint32_t)red[w][om][oc][orr][oln]);
        }
        if constexpr (kFloat) {
            // alpha * acc + beta * C, then bias, ReLU and rounding to D's type
            const bool relu = p.act != 0;
            float x = p.alpha * v;
            if (p.d_type == OUT_BF16) {
                if (p.use_c) x = fmaf(p.beta, from_out_bits<OUT_BF16>(cpre), x);
                __builtin_amdgcn_raw_buffer_store_b16((unsigned short)finish<OUT_BF16>(x, bias, has_bias, relu), rd,
                                                      od, 0, 0);
            } else if (p.d_type == OUT_F16) {
                if (p.use_c) x = fmaf(p.beta, from_out_bits<OUT_F16>(cpre), x);
                __builtin_amdgcn_raw_buffer_store_b16((unsigned short)finish<OUT_F16>(x, bias, has_bias, relu), rd,
                                                      od, 0, 0);
            } else if (p.d_type == OUT_E4M3) {
                if (p.use_c) x = fmaf(p.beta, from_out_bits<OUT_E4M3>(cpre), x);
                __builtin_amdgcn_raw_buffer_store_b8((unsigned char)finish<OUT_E4M3>(x, bias, has_bias, relu), rd,
                                                     od, 0, 0);
            } else if (p.d_type == OUT_E5M2) {
                if (p.use_c) x = fmaf(p.beta, from_out_bits<OUT_E5M2>(cpre), x);
                __builtin_amdgcn_raw_buffer_store_b8((unsigned char)finish<OUT_E5M2>(x, bias, has_bias, relu), rd,
                                                     od, 0, 0);
            } else {
                if (p.use_c) x = fmaf(p.beta, __builtin_bit_cast(float, cpre), x);
                __builtin_amdgcn_raw_buffer_store_b32(finish<OUT_ACC>(x, bias, has_bias, relu), rd, od, 0, 0);
            }
        } else {
            uint32_t x = (uint32_t)p.ialpha * (uint32_t)v;
            if (p.use_c) x += (uint32_t)p.ibeta * cpre;
            __builtin_amdgcn_raw_buffer_store_b32(x, rd, od, 0, 0);
        }
    }
}

template <int DA, int DB>
static hipError_t launch_types(const GemmParams &p, hipStream_t s) {
    typedef Mma16<DA, DB> Op;
    // 8 waves, each with 4 chunks (16 KiB) of copies in flight; 3 chunks (18 KiB) when A has 32 rows
    constexpr int CB = 1, WK = 8;
    const dim3 grid((p.N + 16 * CB - 1) / (16 * CB)), block(WK * 64);
    if (p.M <= 16) hipLaunchKernelGGL((gemm_skinny_kernel<Op, 1, CB, WK, 4>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((gemm_skinny_kernel<Op, 2, CB, WK, 3>), grid, block, 0, s, p);
    return hipGetLastError();
}

hipError_t launch_gemm_skinny(int a, int b, GemmParams p, hipStream_t s) {
    if (p.M > 32) return hipErrorInvalidValue;
    if (a == DT_BF16 && b == DT_BF16) return launch_types<DT_BF16, DT_BF16>(p, s);
    if (a == DT_F16 && b == DT_F16) return launch_types<DT_F16, DT_F16>(p, s);
    if (a == DT_I8 && b == DT_I8) return launch_types<DT_I8, DT_I8>(p, s);
    if (a == DT_E4M3 && b == DT_E4M3) return launch_types<DT_E4M3, DT_E4M3>(p, s);
    if (a == DT_E4M3 && b == DT_E5M2) return launch_types<DT_E4M3, DT_E5M2>(p, s);
    if (a == DT_E5M2 && b == DT_E4M3) return launch_types<DT_E5M2, DT_E4M3>(p, s);
    if (a == DT_E5M2 && b == DT_E5M2) return launch_types<DT_E5M2, DT_E5M2>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace mmac
