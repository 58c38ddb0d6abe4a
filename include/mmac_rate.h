/*
 * mmac_rate -- matrix-instruction rate microbenchmark for MI355X (gfx950).
 *
 * Measures the sustained rate of each matrix instruction the GEMM kernels of
 * libmmac use, issued back to back with no memory traffic on every compute
 * unit, and the shader clock while it runs.  This is the ceiling against
 * which a kernel's fraction of peak is read besides the published one: the
 * pages give an instruction's peak as its operations per cycle times the
 * clock ("CDNA dense MFMA builtins", section "Instruction throughput";
 * "CDNA3 sparse MFMA builtins", section "Instruction throughput", where a
 * sparse instruction's operations count the dense K).  Measurement only: no
 * GEMM goes through this library.
 */
#ifndef MMAC_RATE_H
#define MMAC_RATE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The instructions measured (index for the calls below). */
typedef enum {
    MMAC_RATE_MFMA_BF16 = 0,     /* v_mfma_f32_32x32x16_bf16 */
    MMAC_RATE_MFMA_F16 = 1,      /* v_mfma_f32_32x32x16_f16 */
    MMAC_RATE_MFMA_I8 = 2,       /* v_mfma_i32_32x32x32_i8 */
    MMAC_RATE_MFMA_FP8 = 3,      /* v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 x E5M2 */
    MMAC_RATE_MFMA_FP6 = 4,      /* the same, FP6 E2M3 x BF6 E3M2 */
    MMAC_RATE_MFMA_FP4 = 5,      /* the same, FP4 E2M1 x FP4 E2M1 */
    MMAC_RATE_SMFMAC_F16 = 6,    /* v_smfmac_f32_32x32x32_f16 (4:2 sparse A) */
    MMAC_RATE_SMFMAC_BF16 = 7,   /* v_smfmac_f32_32x32x32_bf16 */
    MMAC_RATE_SMFMAC_I8 = 8,     /* v_smfmac_i32_32x32x64_i8 */
    MMAC_RATE_SMFMAC_FP8 = 9,    /* v_smfmac_f32_32x32x64_fp8_bf8 */
    MMAC_RATE_MFMA_BF16_16 = 10, /* v_mfma_f32_16x16x32_bf16 (the skinny kernel's) */
    MMAC_RATE_COUNT = 11
} mmac_rate_instr_t;

/* Operations of one instruction (2*M*N*K, K the dense K for sparse ones); 0 for an unknown index. */
int64_t mmac_rate_ops(int instr);

/* Static name of an instruction (NULL for an unknown index). */
const char *mmac_rate_name(int instr);

/*
 * Enqueue one measurement on `stream` (a hipStream_t): `blocks` workgroups of
 * MMAC_RATE_WAVES waves each; every wave issues `iters` x MMAC_RATE_CHAINS
 * instructions, in MMAC_RATE_CHAINS independent accumulator chains.
 *   clocks  device memory, 2 * blocks uint64: per workgroup, the shader-clock
 *           cycles (clock64) and the constant-rate ticks (wall_clock64, at
 *           hipDeviceAttributeWallClockRate kHz) its first wave spent in the loop.
 *   sink    device memory, blocks * 64 * MMAC_RATE_WAVES floats that receive
 *           the accumulators (keeps the work observable).
 * Returns 0, -1 for bad arguments (unknown instr, iters < 1, blocks < 1,
 * NULL pointers), or the HIP launch error.
 */
#define MMAC_RATE_WAVES 4
#define MMAC_RATE_CHAINS 4
int mmac_rate_run(int instr, int64_t iters, int blocks, uint64_t *clocks, float *sink, void *stream);

/*
 * The same with a choice of operand data.  random_operands = 0: constant
 * operands (as mmac_rate_run: every instruction multiplies the same small
 * values); 1: random operands, drawn once per wave at the start (random sign
 * and mantissa, exponents around 1 for the floating formats, raw bits for
 * int8 and the 4- / 6-bit formats), each instruction of a loop trip taking A
 * operand c of MMAC_RATE_CHAINS and B operand c mod 2, so the matrix unit's
 * inputs change from one instruction to the next as a GEMM's fragments do.
 * The chip's power management sets a lower clock for switching data than
 * for constant data; this measures the rate a GEMM on random inputs can
 * reach.  Returns as mmac_rate_run; -1 also for random_operands not 0 or 1.
 */
int mmac_rate_run_data(int instr, int random_operands, int64_t iters, int blocks, uint64_t *clocks, float *sink,
                       void *stream);

/* Rate of the constant-rate clock behind the wall ticks (kHz) of the current device; -1 on a HIP
 * error.  A workgroup's shader clock is then cycles / ticks * this rate. */
int64_t mmac_rate_wall_clock_khz(void);

#ifdef __cplusplus
}
#endif

#endif /* MMAC_RATE_H */
