"""Matrix-instruction rate microbenchmark (libmmac_rate.so, include/mmac_rate.h).

measure(instr) issues one matrix instruction back to back on every compute
unit for a fixed time (default 150 ms) and returns its sustained rate and the
shader clock meanwhile: the ceiling a GEMM kernel built on that instruction
can reach on this chip at the clock it actually holds, next to the published
peak (operations per cycle times 2.4 GHz).  With random=True the operands are
random and change from one instruction to the next, as a GEMM's do; the chip
then holds a lower clock than for constant operands.  Measurement only.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmmac_rate.so")
WAVES, CHAINS = 4, 4                      # MMAC_RATE_WAVES, MMAC_RATE_CHAINS

(MFMA_BF16, MFMA_F16, MFMA_I8, MFMA_FP8, MFMA_FP6, MFMA_FP4, SMFMAC_F16, SMFMAC_BF16, SMFMAC_I8, SMFMAC_FP8,
 MFMA_BF16_16) = range(11)
COUNT = 11

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m sparse_matrix_multiply_amd.build` first")
        L = ctypes.CDLL(LIB_PATH)
        L.mmac_rate_ops.restype = ctypes.c_int64
        L.mmac_rate_ops.argtypes = [ctypes.c_int]
        L.mmac_rate_name.restype = ctypes.c_char_p
        L.mmac_rate_name.argtypes = [ctypes.c_int]
        L.mmac_rate_run.restype = ctypes.c_int
        L.mmac_rate_run.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p]
        L.mmac_rate_wall_clock_khz.restype = ctypes.c_int64
        L.mmac_rate_wall_clock_khz.argtypes = []
        L.mmac_rate_run_data.restype = ctypes.c_int
        L.mmac_rate_run_data.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p]
        _lib = L
    return _lib


def name(instr):
    return lib().mmac_rate_name(instr).decode()


def measure(instr, seconds=0.15, device=None, random=False):
    """Sustained rate of one instruction on the whole GPU, multiplying constant operands or (random)
    random ones that change from one instruction to the next.  Returns a dict: TFLOP/s (TOP/s for
    int8; dense-equivalent for sparse), the shader clock in GHz (each workgroup's clock64 cycles over
    its wall-clock ticks), cycles per instruction per SIMD at that clock, and the duration."""
    dev = torch.device("cuda", 0) if device is None else device
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = 4 * cus                     # four waves per SIMD once all are resident
    clocks = torch.zeros(2 * blocks, dtype=torch.int64, device=dev)
    sink = torch.empty(blocks * 64 * WAVES, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    L = lib()

    def run(iters):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rc = L.mmac_rate_run_data(instr, 1 if random else 0, iters, blocks, ctypes.c_void_p(clocks.data_ptr()),
                                  ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"mmac_rate_run_data({instr}, {int(random)}) failed: {rc}")
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3

    run(1000)                            # warm-up (clocks ramp)
    t = run(2000)
    iters = max(2000, int(2000 * seconds / max(t, 1e-6)))
    t = run(iters)
    c = clocks.view(blocks, 2).double().cpu()
    ops = L.mmac_rate_ops(instr) * iters * CHAINS * WAVES * blocks
    # the workgroups do not all start at once, so the clock comes from each one's own cycles over its
    # own constant-rate ticks, not from the event-timed duration
    khz = L.mmac_rate_wall_clock_khz()
    sclk = float((c[:, 0] / c[:, 1]).mean()) * khz * 1e3 if khz > 0 else float("nan")
    instr_per_simd = iters * CHAINS * WAVES * blocks / (4 * cus)
    return {"instr": name(instr), "TFLOP/s": ops / t / 1e12, "sclk_GHz": sclk / 1e9,
            "cycles_per_instr": sclk * t / instr_per_simd, "seconds": t, "random_operands": bool(random)}
