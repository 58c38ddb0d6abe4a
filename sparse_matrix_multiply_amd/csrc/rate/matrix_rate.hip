// Matrix-instruction rate microbenchmark (include/mmac_rate.h): every wave
// runs MMAC_RATE_CHAINS independent accumulator chains of one instruction,
// back to back, with its operands held in registers (constant, or random bits
// that change from one instruction to the next), and records the shader clock
// cycles and constant-rate ticks it spent.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mmac_rate.h"

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x16 __attribute__((ext_vector_type(16)));

// Operand formats, for drawing operand bits (below).
enum Fmt { F_BF16, F_F16, F_I8, F_E4M3, F_E5M2, F_FP6, F_BF6, F_FP4 };

// Constant operands: small normal values in every format (1.0 and the like), the same in every
// instruction, so the matrix unit's inputs never change.
__device__ __forceinline__ uint32_t const_word(Fmt f) {
    switch (f) {
    case F_BF16: case F_F16: return 0x3c003c00u;     // binary16 1.0 pairs (bfloat16 0x3c00 = 2^-7)
    case F_I8: return 0x01010101u;
    default: return 0x38383838u;                     // E4M3 1.0 / E5M2 0.5 bytes; FP4 / FP6 fields of small values
    }
}

// Random operands: 32 random bits made into elements of the format with a random sign and
// mantissa and an exponent drawn from four values around 1 (|x| in [2^-3, 2^1) or so), as
// normally distributed data has; integer and 4- / 6-bit formats take the bits as they are (every
// code is finite).
__device__ __forceinline__ uint32_t random_word(Fmt f, uint32_t r) {
    switch (f) {
    case F_BF16: {   // sign, 7 mantissa bits, exponent 124 + (0..3)
        const uint32_t keep = r & 0x807f807fu, e = (r >> 7) & 0x00030003u;
        return keep | ((e + 0x007c007cu) << 7);
    }
    case F_F16: {    // sign, 10 mantissa bits, exponent 13 + (0..3)
        const uint32_t keep = r & 0x83ff83ffu, e = (r >> 10) & 0x00030003u;
        return keep | ((e + 0x000d000du) << 10);
    }
    case F_E4M3: {   // sign, 3 mantissa bits, exponent 5 + (0..3)
        const uint32_t keep = r & 0x87878787u, e = (r >> 3) & 0x03030303u;
        return keep | ((e + 0x05050505u) << 3);
    }
    case F_E5M2: {   // sign, 2 mantissa bits, exponent 13 + (0..3)
        const uint32_t keep = r & 0x83838383u, e = (r >> 2) & 0x03030303u;
        return keep | ((e + 0x0d0d0d0du) << 2);
    }
    default: return r;
    }
}

// A 32-bit mix of a counter (the finalizer of MurmurHash3).
__device__ __forceinline__ uint32_t mix32(uint32_t h) {
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

// One instruction class: operand A of NA words in format FA, operand B of NB words in format FB.
template <int I> struct Instr;

template <> struct Instr<MMAC_RATE_MFMA_BF16> {
    typedef f32x16 acc_t;
    static constexpr int NA = 4, NB = 4;
    static constexpr Fmt FA = F_BF16, FB = F_BF16;
    static __device__ __forceinline__ acc_t run(acc_t c, const i32x4 &a, const i32x4 &b) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                      0, 0, 0);
    }
};
template <> struct Instr<MMAC_RATE_MFMA_F16> {
    typedef f32x16 acc_t;
    static constexpr int NA = 4, NB = 4;
    static constexpr Fmt FA = F_F16, FB = F_F16;
    static __device__ __forceinline__ acc_t run(acc_t c, const i32x4 &a, const i32x4 &b) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                     0, 0, 0);
    }
};
template <> struct Instr<MMAC_RATE_MFMA_I8> {
    typedef i32x16 acc_t;
    static constexpr int NA = 4, NB = 4;
    static constexpr Fmt FA = F_I8, FB = F_I8;
    static __device__ __forceinline__ acc_t run(acc_t c, const i32x4 &a, const i32x4 &b) {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
    }
};
template <int FMT_A, int FMT_B, Fmt FA_, Fmt FB_> struct InstrF8F6F4 {
    typedef f32x16 acc_t;
    static constexpr int NA = 8, NB = 8;
    static constexpr Fmt FA = FA_, FB = FB_;
    static __device__ __forceinline__ acc_t run(acc_t c, const i32x8 &a, const i32x8 &b) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT_A, FMT_B, 0, 127, 0, 127);
    }
};
template <> struct Instr<MMAC_RATE_MFMA_FP8> : InstrF8F6F4<0, 1, F_E4M3, F_E5M2> {};
template <> struct Instr<MMAC_RATE_MFMA_FP6> : InstrF8F6F4<2, 3, F_FP6, F_BF6> {};
template <> struct Instr<MMAC_RATE_MFMA_FP4> : InstrF8F6F4<4, 4, F_FP4, F_FP4> {};
template <> struct Instr<MMAC_RATE_SMFMAC_F16> {
    typedef f32x16 acc_t;
    static constexpr int NA = 4, NB = 8;
    static constexpr Fmt FA = F_F16, FB = F_F16;
    static __device__ __forceinline__ acc_t run(acc_t c, const i32x4 &a, const i32x8 &b) {
        return __builtin_amdgcn_smfmac_f32_32x32x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x16, b), c,
                                                       0x8888, 0, 0);
    }
};
template <> struct Instr<MMAC_RATE_SMFMAC_BF16> {
    typedef f32x16 acc_t;
    static constexpr int NA = 4, NB = 8;
    static constexpr Fmt FA = F_BF16, FB = F_BF16;
    static __device__ __forceinline__ acc_t run(acc_t c, const i32x4 &a, const i32x8 &b) {
        return __builtin_amdgcn_smfmac_f32_32x32x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x16, b),
                                                        c, 0x8888, 0, 0);
    }
};
template <> struct Instr<MMAC_RATE_SMFMAC_I8> {
    typedef i32x16 acc_t;
    static constexpr int NA = 4, NB = 8;
    static constexpr Fmt FA = F_I8, FB = F_I8;
    static __device__ __forceinline__ acc_t run(acc_t c, const i32x4 &a, const i32x8 &b) {
        return __builtin_amdgcn_smfmac_i32_32x32x64_i8(a, b, c, (int)0x88888888, 0, 0);
    }
};
template <> struct Instr<MMAC_RATE_SMFMAC_FP8> {
    typedef f32x16 acc_t;
    static constexpr int NA = 4, NB = 8;
    static constexpr Fmt FA = F_E4M3, FB = F_E5M2;
    static __device__ __forceinline__ acc_t run(acc_t c, const i32x4 &a, const i32x8 &b) {
        return __builtin_amdgcn_smfmac_f32_32x32x64_fp8_bf8(a, b, c, (int)0x88888888, 0, 0);
    }
};
template <> struct Instr<MMAC_RATE_MFMA_BF16_16> {
    typedef f32x4 acc_t;
    static constexpr int NA = 4, NB = 4;
    static constexpr Fmt FA = F_BF16, FB = F_BF16;
    static __device__ __forceinline__ acc_t run(acc_t c, const i32x4 &a, const i32x4 &b) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                      0, 0, 0);
    }
};

template <int N> struct Words;
template <> struct Words<4> { typedef i32x4 type; };
template <> struct Words<8> { typedef i32x8 type; };

// Operands a wave holds: instruction c of a loop trip takes A operand c and B operand c mod 2.
// With constant operands every one is the constant pattern, with one lane-dependent bit the
// compiler cannot fold; with random operands every operand, lane and word has bits of its own,
// so each instruction's inputs differ from those of the instruction before (as the fragments of a
// GEMM's step do), at a register cost that keeps four waves on every SIMD.
constexpr int kSetsA = MMAC_RATE_CHAINS, kSetsB = 2;

template <int N>
__device__ __forceinline__ typename Words<N>::type make_operand(Fmt f, bool random, uint32_t seed, int x) {
    typename Words<N>::type v;
#pragma unroll
    for (int w = 0; w < N; ++w) {
        const uint32_t r = mix32(seed * 0x9e3779b9u + (uint32_t)w * 0x632be5abu + 0x1234567u);
        v[w] = (int)(random ? random_word(f, r) : const_word(f) ^ (w == 0 ? (uint32_t)x : 0u));
    }
    return v;
}

template <int I>
__global__ __launch_bounds__(64 * MMAC_RATE_WAVES) void rate_kernel(int random, int64_t iters, uint64_t *clocks,
                                                                    float *sink) {
    typedef Instr<I> In;
    typedef typename In::acc_t acc_t;
    typedef typename Words<In::NA>::type a_t;
    typedef typename Words<In::NB>::type b_t;
    acc_t acc[MMAC_RATE_CHAINS];
#pragma unroll
    for (int c = 0; c < MMAC_RATE_CHAINS; ++c) acc[c] = acc_t{};
    const int x = (int)(threadIdx.x & 1);     // a lane-dependent operand bit the compiler cannot fold
    const uint32_t lane_id = blockIdx.x * blockDim.x + threadIdx.x;
    a_t a[kSetsA];
    b_t b[kSetsB];
#pragma unroll
    for (int s = 0; s < kSetsA; ++s) a[s] = make_operand<In::NA>(In::FA, random != 0, lane_id * 8 + s, x);
#pragma unroll
    for (int s = 0; s < kSetsB; ++s) b[s] = make_operand<In::NB>(In::FB, random != 0, lane_id * 8 + 4 + s, x);
    const uint64_t t0 = clock64(), w0 = wall_clock64();
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < MMAC_RATE_CHAINS; ++c) acc[c] = In::run(acc[c], a[c], b[c % kSetsB]);
    }
    const uint64_t t1 = clock64(), w1 = wall_clock64();
    if (threadIdx.x == 0) {
        clocks[2 * blockIdx.x] = t1 - t0;
        clocks[2 * blockIdx.x + 1] = w1 - w0;
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < MMAC_RATE_CHAINS; ++c) s += (float)acc[c][0];
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

template <int I>
hipError_t launch(int random, int64_t iters, int blocks, uint64_t *clocks, float *sink, hipStream_t s) {
    hipLaunchKernelGGL(rate_kernel<I>, dim3(blocks), dim3(64 * MMAC_RATE_WAVES), 0, s, random, iters, clocks, sink);
    return hipGetLastError();
}

}  // namespace

extern "C" {

int64_t mmac_rate_ops(int instr) {
    switch (instr) {
    case MMAC_RATE_MFMA_BF16: case MMAC_RATE_MFMA_F16: return 2LL * 32 * 32 * 16;
    case MMAC_RATE_MFMA_I8: return 2LL * 32 * 32 * 32;
    case MMAC_RATE_MFMA_FP8: case MMAC_RATE_MFMA_FP6: case MMAC_RATE_MFMA_FP4: return 2LL * 32 * 32 * 64;
    case MMAC_RATE_SMFMAC_F16: case MMAC_RATE_SMFMAC_BF16: return 2LL * 32 * 32 * 32;
    case MMAC_RATE_SMFMAC_I8: case MMAC_RATE_SMFMAC_FP8: return 2LL * 32 * 32 * 64;
    case MMAC_RATE_MFMA_BF16_16: return 2LL * 16 * 16 * 32;
    default: return 0;
    }
}

const char *mmac_rate_name(int instr) {
    static const char *const names[MMAC_RATE_COUNT] = {
        "v_mfma_f32_32x32x16_bf16", "v_mfma_f32_32x32x16_f16", "v_mfma_i32_32x32x32_i8",
        "v_mfma_scale_f32_32x32x64_f8f6f4 (fp8 x bf8)", "v_mfma_scale_f32_32x32x64_f8f6f4 (fp6 x bf6)",
        "v_mfma_scale_f32_32x32x64_f8f6f4 (fp4 x fp4)", "v_smfmac_f32_32x32x32_f16", "v_smfmac_f32_32x32x32_bf16",
        "v_smfmac_i32_32x32x64_i8", "v_smfmac_f32_32x32x64_fp8_bf8", "v_mfma_f32_16x16x32_bf16"};
    return instr >= 0 && instr < MMAC_RATE_COUNT ? names[instr] : nullptr;
}

int mmac_rate_run_data(int instr, int random_operands, int64_t iters, int blocks, uint64_t *clocks, float *sink,
                       void *stream) {
    if (iters < 1 || blocks < 1 || !clocks || !sink || (random_operands != 0 && random_operands != 1)) return -1;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int r = random_operands;
    switch (instr) {
    case MMAC_RATE_MFMA_BF16: return launch<MMAC_RATE_MFMA_BF16>(r, iters, blocks, clocks, sink, s);
    case MMAC_RATE_MFMA_F16: return launch<MMAC_RATE_MFMA_F16>(r, iters, blocks, clocks, sink, s);
    case MMAC_RATE_MFMA_I8: return launch<MMAC_RATE_MFMA_I8>(r, iters, blocks, clocks, sink, s);
    case MMAC_RATE_MFMA_FP8: return launch<MMAC_RATE_MFMA_FP8>(r, iters, blocks, clocks, sink, s);
    case MMAC_RATE_MFMA_FP6: return launch<MMAC_RATE_MFMA_FP6>(r, iters, blocks, clocks, sink, s);
    case MMAC_RATE_MFMA_FP4: return launch<MMAC_RATE_MFMA_FP4>(r, iters, blocks, clocks, sink, s);
    case MMAC_RATE_SMFMAC_F16: return launch<MMAC_RATE_SMFMAC_F16>(r, iters, blocks, clocks, sink, s);
    case MMAC_RATE_SMFMAC_BF16: return launch<MMAC_RATE_SMFMAC_BF16>(r, iters, blocks, clocks, sink, s);
    case MMAC_RATE_SMFMAC_I8: return launch<MMAC_RATE_SMFMAC_I8>(r, iters, blocks, clocks, sink, s);
    case MMAC_RATE_SMFMAC_FP8: return launch<MMAC_RATE_SMFMAC_FP8>(r, iters, blocks, clocks, sink, s);
    case MMAC_RATE_MFMA_BF16_16: return launch<MMAC_RATE_MFMA_BF16_16>(r, iters, blocks, clocks, sink, s);
    default: return -1;
    }
}

int mmac_rate_run(int instr, int64_t iters, int blocks, uint64_t *clocks, float *sink, void *stream) {
    return mmac_rate_run_data(instr, 0, iters, blocks, clocks, sink, stream);
}

int64_t mmac_rate_wall_clock_khz(void) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
        return -1;
    return khz;
}

}  // extern "C"
