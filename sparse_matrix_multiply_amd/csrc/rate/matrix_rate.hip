// Matrix-instruction rate microbenchmark (include/mmac_rate.h): every wave
// runs MMAC_RATE_CHAINS independent accumulator chains of one instruction,
// back to back, with its operands held in registers, and records the shader
// clock cycles and constant-rate ticks it spent.
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

// Operand bit patterns: small normal values in every format (the instructions' timing does not
// depend on the data; NaNs and subnormals are avoided anyway).
constexpr int kOne16 = 0x3c003c00;     // binary16 1.0 pairs (bfloat16 0x3c00 = 2^-7)
constexpr int kOne8 = 0x38383838;      // E4M3 1.0 / E5M2 0.5 bytes; FP4 / FP6 fields of small values

template <int I> struct Instr;

template <> struct Instr<MMAC_RATE_MFMA_BF16> {
    typedef f32x16 acc_t;
    static __device__ __forceinline__ acc_t run(acc_t c, int x) {
        const i32x4 v = {kOne16 ^ x, kOne16, kOne16, kOne16};
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v), __builtin_bit_cast(bf16x8, v), c,
                                                      0, 0, 0);
    }
};
template <> struct Instr<MMAC_RATE_MFMA_F16> {
    typedef f32x16 acc_t;
    static __device__ __forceinline__ acc_t run(acc_t c, int x) {
        const i32x4 v = {kOne16 ^ x, kOne16, kOne16, kOne16};
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, v), __builtin_bit_cast(f16x8, v), c,
                                                     0, 0, 0);
    }
};
template <> struct Instr<MMAC_RATE_MFMA_I8> {
    typedef i32x16 acc_t;
    static __device__ __forceinline__ acc_t run(acc_t c, int x) {
        const i32x4 v = {0x01010101 ^ x, 0x01010101, 0x01010101, 0x01010101};
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(v, v, c, 0, 0, 0);
    }
};
template <int FMT_A, int FMT_B> struct InstrF8F6F4 {
    typedef f32x16 acc_t;
    static __device__ __forceinline__ acc_t run(acc_t c, int x) {
        const i32x8 v = {kOne8 ^ x, kOne8, kOne8, kOne8, kOne8, kOne8, kOne8, kOne8};
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v, v, c, FMT_A, FMT_B, 0, 127, 0, 127);
    }
};
template <> struct Instr<MMAC_RATE_MFMA_FP8> : InstrF8F6F4<0, 1> {};
template <> struct Instr<MMAC_RATE_MFMA_FP6> : InstrF8F6F4<2, 3> {};
template <> struct Instr<MMAC_RATE_MFMA_FP4> : InstrF8F6F4<4, 4> {};
template <> struct Instr<MMAC_RATE_SMFMAC_F16> {
    typedef f32x16 acc_t;
    static __device__ __forceinline__ acc_t run(acc_t c, int x) {
        const i32x4 a = {kOne16 ^ x, kOne16, kOne16, kOne16};
        const i32x8 b = {kOne16, kOne16, kOne16, kOne16, kOne16, kOne16, kOne16, kOne16};
        return __builtin_amdgcn_smfmac_f32_32x32x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x16, b), c,
                                                       0x8888, 0, 0);
    }
};
template <> struct Instr<MMAC_RATE_SMFMAC_BF16> {
    typedef f32x16 acc_t;
    static __device__ __forceinline__ acc_t run(acc_t c, int x) {
        const i32x4 a = {kOne16 ^ x, kOne16, kOne16, kOne16};
        const i32x8 b = {kOne16, kOne16, kOne16, kOne16, kOne16, kOne16, kOne16, kOne16};
        return __builtin_amdgcn_smfmac_f32_32x32x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x16, b),
                                                        c, 0x8888, 0, 0);
    }
};
template <> struct Instr<MMAC_RATE_SMFMAC_I8> {
    typedef i32x16 acc_t;
    static __device__ __forceinline__ acc_t run(acc_t c, int x) {
        const i32x4 a = {0x01010101 ^ x, 0x01010101, 0x01010101, 0x01010101};
        const i32x8 b = {0x01010101, 0x01010101, 0x01010101, 0x01010101, 0x01010101, 0x01010101, 0x01010101,
                         0x01010101};
        return __builtin_amdgcn_smfmac_i32_32x32x64_i8(a, b, c, (int)0x88888888, 0, 0);
    }
};
template <> struct Instr<MMAC_RATE_SMFMAC_FP8> {
    typedef f32x16 acc_t;
    static __device__ __forceinline__ acc_t run(acc_t c, int x) {
        const i32x4 a = {kOne8 ^ x, kOne8, kOne8, kOne8};
        const i32x8 b = {kOne8, kOne8, kOne8, kOne8, kOne8, kOne8, kOne8, kOne8};
        return __builtin_amdgcn_smfmac_f32_32x32x64_fp8_bf8(a, b, c, (int)0x88888888, 0, 0);
    }
};
template <> struct Instr<MMAC_RATE_MFMA_BF16_16> {
    typedef f32x4 acc_t;
    static __device__ __forceinline__ acc_t run(acc_t c, int x) {
        const i32x4 v = {kOne16 ^ x, kOne16, kOne16, kOne16};
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), __builtin_bit_cast(bf16x8, v), c,
                                                      0, 0, 0);
    }
};

template <int I>
__global__ __launch_bounds__(64 * MMAC_RATE_WAVES) void rate_kernel(int64_t iters, uint64_t *clocks, float *sink) {
    typedef typename Instr<I>::acc_t acc_t;
    acc_t acc[MMAC_RATE_CHAINS];
#pragma unroll
    for (int c = 0; c < MMAC_RATE_CHAINS; ++c) acc[c] = acc_t{};
    const int x = (int)(threadIdx.x & 1);     // a lane-dependent operand bit the compiler cannot fold
    const uint64_t t0 = clock64(), w0 = wall_clock64();
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < MMAC_RATE_CHAINS; ++c) acc[c] = Instr<I>::run(acc[c], x);
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
hipError_t launch(int64_t iters, int blocks, uint64_t *clocks, float *sink, hipStream_t s) {
    hipLaunchKernelGGL(rate_kernel<I>, dim3(blocks), dim3(64 * MMAC_RATE_WAVES), 0, s, iters, clocks, sink);
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

int mmac_rate_run(int instr, int64_t iters, int blocks, uint64_t *clocks, float *sink, void *stream) {
    if (iters < 1 || blocks < 1 || !clocks || !sink) return -1;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    switch (instr) {
    case MMAC_RATE_MFMA_BF16: return launch<MMAC_RATE_MFMA_BF16>(iters, blocks, clocks, sink, s);
    case MMAC_RATE_MFMA_F16: return launch<MMAC_RATE_MFMA_F16>(iters, blocks, clocks, sink, s);
    case MMAC_RATE_MFMA_I8: return launch<MMAC_RATE_MFMA_I8>(iters, blocks, clocks, sink, s);
    case MMAC_RATE_MFMA_FP8: return launch<MMAC_RATE_MFMA_FP8>(iters, blocks, clocks, sink, s);
    case MMAC_RATE_MFMA_FP6: return launch<MMAC_RATE_MFMA_FP6>(iters, blocks, clocks, sink, s);
    case MMAC_RATE_MFMA_FP4: return launch<MMAC_RATE_MFMA_FP4>(iters, blocks, clocks, sink, s);
    case MMAC_RATE_SMFMAC_F16: return launch<MMAC_RATE_SMFMAC_F16>(iters, blocks, clocks, sink, s);
    case MMAC_RATE_SMFMAC_BF16: return launch<MMAC_RATE_SMFMAC_BF16>(iters, blocks, clocks, sink, s);
    case MMAC_RATE_SMFMAC_I8: return launch<MMAC_RATE_SMFMAC_I8>(iters, blocks, clocks, sink, s);
    case MMAC_RATE_SMFMAC_FP8: return launch<MMAC_RATE_SMFMAC_FP8>(iters, blocks, clocks, sink, s);
    case MMAC_RATE_MFMA_BF16_16: return launch<MMAC_RATE_MFMA_BF16_16>(iters, blocks, clocks, sink, s);
    default: return -1;
    }
}

}  // extern "C"
