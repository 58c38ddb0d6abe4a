"""Benchmark: dense bf16, dense fp8 and 4:2-sparse fp8 GEMM at 8192^3 on one MI355X.

One step is one pass of the whole path over one batch of synthetic input:
  1. 4:2 compression of the pruned fp8 A (mmac_sparse24_compress),
  2. sparse fp8 x bf8 GEMM on it (mmac_gemm_sparse24),
  3. dense bf16 GEMM, D = A*B + C (mmac_gemm_dense),
  4. dense fp8 E4M3 x bf8 E5M2 GEMM (mmac_gemm_dense).
The inputs are resident in HBM before timing starts.  `value` is the step's
work (2*M*N*K per GEMM, dense-equivalent K for the sparse one) divided by the
wall time of the step.  Each kernel is also timed with HIP events on the
stream it runs on, and the slowest one is reported against its roofline: the
published peak, and the sustained rate of its matrix instruction measured on
this GPU by the rate microbenchmark (`matrix_rates`) with random operands, as
the GEMM's are (the chip holds a lower clock for them than for constant ones;
both rates and clocks are in the line).  The CPU oracle is timed on a bounded
slice of the bf16 GEMM (`cpu_baseline`).  `configs` gives every smaller
workload at its full size -- 256^3 bf16, 1024^3 int8, 4096^3 bf16,
16x4096x4096 bf16 and the 4:2 fp16 4096x4096x8192 compress + GEMM -- with its
GPU time, a full comparison with the oracle, and the oracle's own wall time on
the host cores (the first two also on one thread).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-check]
                       [--no-configs] [--no-rates] [--suite]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s + % MFMA peak, bf16/fp8 dense and 4:2 sparse at 8192³, 1 GPU"
# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp8": 5000.0, "int8": 5000.0, "fp6": 10100.0, "fp4": 10100.0}
PEAK_HBM_GBS = 8000.0


# Source files each kernel is built from: the HBM traffic recorded in profiles/traffic_8192.json
# applies only while their hash is the one recorded there.
_KSRC = {
    "dense": ["include/mmac.h", "sparse_matrix_multiply_amd/csrc/device.h", "sparse_matrix_multiply_amd/csrc/gemm_tiled.h",
              "sparse_matrix_multiply_amd/csrc/launch.h", "sparse_matrix_multiply_amd/csrc/tiles_dense.h",
              "sparse_matrix_multiply_amd/csrc/inst/dense_bf16.hip",
              "sparse_matrix_multiply_amd/csrc/inst/dense_e4m3_e5m2.hip", "sparse_matrix_multiply_amd/csrc/abi.hip"],
    "sparse": ["include/mmac.h", "sparse_matrix_multiply_amd/csrc/device.h", "sparse_matrix_multiply_amd/csrc/gemm_tiled.h",
               "sparse_matrix_multiply_amd/csrc/launch.h", "sparse_matrix_multiply_amd/csrc/tiles_sparse.h",
               "sparse_matrix_multiply_amd/csrc/inst/sparse_e4m3_e5m2.hip", "sparse_matrix_multiply_amd/csrc/abi.hip"],
    "compress": ["include/mmac.h", "sparse_matrix_multiply_amd/csrc/device.h", "sparse_matrix_multiply_amd/csrc/launch.h",
                 "sparse_matrix_multiply_amd/csrc/compress.hip", "sparse_matrix_multiply_amd/csrc/abi.hip"],
}
# kernel names of the launches this benchmark makes (default tile choice at 8192^3)
# kernel-name prefixes in the profile summary (the stage count and other trailing
# template arguments may change without renaming the part)
_KNAME = {"dense_bf16": ("dense", "gemm_tiled_kernel<mmac::MmaDense16<2>, 256, 256,"),
          "dense_fp8": ("dense", "gemm_tiled_kernel<mmac::MmaDenseF8<0, 1>, 256, 256,"),
          "sparse_fp8": ("sparse", "gemm_tiled_kernel<mmac::MmaSparse8<4, 5>, 256, 256,"),
          "compress_fp8": ("compress", "compress_kernel<4, false>")}


def _code_only(text):
    """C/C++ source without its comments and with whitespace runs collapsed: what the compiler sees,
    so that a change to a comment does not count as a change of the kernel."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash(files):
    """First 16 hex digits of the SHA-256 of the files' code (comments and layout ignored)."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(part):
    """HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE) recorded by the last counter runs,
    or None when the kernel's sources changed since (or nothing was recorded)."""
    kind, name = _KNAME[part]
    try:
        kernels = json.load(open(os.path.join(ROOT, "profiles", "traffic_8192.json")))["kernels"]
        rec = next(v for k, v in kernels.items() if k.startswith(name))
    except (OSError, KeyError, ValueError, StopIteration):
        return None
    if source_hash(_KSRC[kind]) != rec["source_hash"]:
        return None
    return {"bytes": rec["fetch_bytes"] + rec["write_bytes"], "read_bytes": rec["fetch_bytes"],
            "write_bytes": rec["write_bytes"],
            "algorithmic_bytes": rec["algorithmic_read_bytes"] + rec["algorithmic_write_bytes"]}


def gemm_flops(M, N, K):
    """Work of one GEMM: 2*M*N*K operations (for a 4:2-sparse A, K is the dense K)."""
    return 2 * int(M) * int(N) * int(K)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration section (GPU time, full oracle check and oracle time of "
                         "the 256^3, 1024^3 int8, 4096^3, 16x4096x4096 and 4:2 fp16 workloads)")
    ap.add_argument("--no-rates", action="store_true",
                    help="skip the matrix-instruction rate microbenchmark and the all-ones run of the bf16 GEMM "
                         "(the context beside the roofline; counter runs of the step use this)")
    ap.add_argument("--cpu-rows", type=int, default=0, help="rows of the oracle slice (0 = calibrate)")
    ap.add_argument("--suite", action="store_true",
                    help="instead of the step, time every workload once (one JSON line with a 'suite' object)")
    ap.add_argument("--only", choices=["skinny", "compress_fp8", "rates", "bf16_8192", "bf16_8192_ones"], default=None,
                    help="only run one kernel --steps times after --warmup (for counter runs): the 16x4096x4096 "
                         "bf16 skinny GEMM (beta = 1, B and D rotated through 16 copies past the Infinity Cache), "
                         "the 8192^2 fp8 4:2 compressor (8 copies rotated), the matrix-rate microbenchmark, or the "
                         "8192^3 bf16 GEMM (beta = 1) on its random inputs or on all-ones A and B")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain elementwise copy of this many MiB (fp32) three times: the known-size "
                         "kernel that calibrates the FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def copy_probe(mib):
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        torch.mul(x, 2.0, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe": {"bytes_read": n * 4, "bytes_written": n * 4, "launches": 3}}))


def main():
    args = parse()
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    if args.suite:
        suite()
        return
    if args.only:
        only(args.only, args.steps, args.warmup)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_matrix_multiply_amd as mm
    import workloads as W

    mm.lib()                                  # fail loudly if the HIP library is missing
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    F16, BF16, I8, E4M3, E5M2 = W.F16, W.BF16, W.I8, W.E4M3, W.E5M2

    def to_dev(bits, t):
        host = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16 if bits.dtype == np.uint16 else np.int8))
        x = host.to(dev)
        return x.view({BF16: torch.bfloat16, F16: torch.float16, E4M3: torch.float8_e4m3fn,
                       E5M2: torch.float8_e5m2}[t])

    t_gen = time.perf_counter()
    wb = W.workload("bf16_8192")
    w8 = W.workload("fp8_8192")
    ws = W.workload("fp8_8192_sparse")
    M = N = K = 8192
    Ab, Bb, Cb = to_dev(wb["A"], BF16), to_dev(wb["B"], BF16), torch.from_numpy(wb["C"]).to(dev)
    A8, B8 = to_dev(w8["A"], E4M3), to_dev(w8["B"], E5M2)
    As = to_dev(ws["A"], E4M3)
    Db = torch.empty((M, N), dtype=torch.float32, device=dev)
    D8 = torch.empty((M, N), dtype=torch.float32, device=dev)
    Ds = torch.empty((M, N), dtype=torch.float32, device=dev)
    Ac = torch.empty((M, K // 2), dtype=torch.float8_e4m3fn, device=dev)
    idx = torch.empty((M, K // 32), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    print(f"# inputs ready in {t_gen:.1f} s", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    parts = ["compress_fp8", "sparse_fp8", "dense_bf16", "dense_fp8"]

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        mm.sparse24_compress(As, Ac, idx, a_type=E4M3, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        mm.gemm_sparse24(Ac, idx, B8, Ds, K=K, alpha=1.0, beta=0.0, a_type=E4M3, b_type=E5M2, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        mm.gemm_dense(Ab, Bb, Db, 1.0, 1.0, Cb, a_type=BF16, b_type=BF16, stream=stream)
        if ev is not None:
            ev[3].record(stream)
        mm.gemm_dense(A8, B8, D8, 1.0, 0.0, None, a_type=E4M3, b_type=E5M2, stream=stream)
        if ev is not None:
            ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    part_ms = {p: 0.0 for p in parts}
    for ev in events:
        for q, p in enumerate(parts):
            part_ms[p] += ev[q].elapsed_time(ev[q + 1]) / args.steps

    flops = {"compress_fp8": 0, "sparse_fp8": gemm_flops(M, N, K), "dense_bf16": gemm_flops(M, N, K),
             "dense_fp8": gemm_flops(M, N, K)}
    step_flops = sum(flops.values())
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    # sparse: dense-equivalent FLOP against 2x the dense peak == effective FLOP against the dense peak
    peak = {"sparse_fp8": 2 * PEAK_TFLOPS["fp8"], "dense_bf16": PEAK_TFLOPS["bf16"], "dense_fp8": PEAK_TFLOPS["fp8"]}
    comp_bytes = M * K + M * (K // 2) + M * (K // 32) * 4        # read A, write Ac + idx
    report = {}
    for p in parts:
        t = part_ms[p] * 1e-3
        if p == "compress_fp8":
            report[p] = {"ms": round(part_ms[p], 4), "GB/s": round(comp_bytes / t / 1e9, 1),
                         "frac_hbm_peak": round(comp_bytes / t / 1e9 / PEAK_HBM_GBS, 4)}
        else:
            tf = flops[p] / t / 1e12
            r = {"ms": round(part_ms[p], 4), "TFLOP/s": round(tf, 1), "frac_peak": round(tf / peak[p], 4)}
            if p == "sparse_fp8":
                r["TFLOP/s_dense_equivalent"] = r.pop("TFLOP/s")
                r["TFLOP/s_effective"] = round(tf / 2, 1)
            report[p] = r

    dominant = max(parts, key=lambda p: part_ms[p])
    if dominant == "compress_fp8":
        roof = {"bound": "hbm", "achieved": round(comp_bytes / (part_ms[dominant] * 1e-3) / 1e9, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        ach = flops[dominant] / (part_ms[dominant] * 1e-3) / 1e12
        if dominant == "sparse_fp8":
            ach /= 2                                  # effective FLOP vs the dense fp8 peak
        pk = PEAK_TFLOPS["bf16" if dominant == "dense_bf16" else "fp8"]
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": pk, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["kernel"] = dominant
    tr = measured_traffic(dominant)
    roof["traffic"] = tr["bytes"] if tr else None
    roof["traffic_kind"] = ("bytes the L2 caches read from and wrote to the memory fabric per launch (TCC FETCH_SIZE and "
                            "WRITE_SIZE, calibrated on a 1 GiB copy); Infinity Cache hits are included: no counter on "
                            "gfx950 separates HBM from Infinity Cache traffic")
    if tr:
        roof["traffic_detail"] = tr

    # the sustained rate of the dominant kernel's instruction on random operands (as the GEMM's inputs
    # are), measured on this GPU, beside the published peak; the constant-operand rate for reference
    rates = None
    if not args.no_rates:
        rates = matrix_rates()
        key = {"dense_bf16": "bf16_mfma", "dense_fp8": "fp8_mfma", "sparse_fp8": "fp8_smfmac"}.get(dominant)
        if key in rates:
            half = 2 if dominant == "sparse_fp8" else 1
            rnd, cst = rates[key]["random_operands"], rates[key]["constant_operands"]
            roof["sustained_peak"] = round(rnd["TFLOP/s"] / half, 1)
            roof["sustained_sclk_MHz"] = rnd["sclk_MHz"]
            roof["frac_of_sustained"] = round(roof["achieved"] / roof["sustained_peak"], 4)
            roof["sustained_peak_constant_operands"] = round(cst["TFLOP/s"] / half, 1)
            roof["sustained_note"] = ("sustained_peak: the instruction alone, back to back on every SIMD, on random "
                                      "operands that change from one instruction to the next; the chip's power "
                                      "management holds a lower clock for them than for constant operands")
    # the same bf16 GEMM (same shape, beta = 1, same C) on all-ones A and B: the kernel is unchanged,
    # only the data the matrix units switch is; context for the power-limited clock, not the metric
    if dominant == "dense_bf16" and not args.no_rates:
        ones_a = torch.ones((M, K), dtype=torch.bfloat16, device=dev)
        ones_b = torch.ones((N, K), dtype=torch.bfloat16, device=dev)
        for _ in range(3):
            mm.gemm_dense(ones_a, ones_b, Db, 1.0, 1.0, Cb, a_type=BF16, b_type=BF16, stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            mm.gemm_dense(ones_a, ones_b, Db, 1.0, 1.0, Cb, a_type=BF16, b_type=BF16, stream=stream)
        e1.record(stream)
        e1.synchronize()
        ones_tf = gemm_flops(M, N, K) / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e12
        roof["achieved_constant_operands"] = round(ones_tf, 1)
        roof["frac_constant_operands"] = round(ones_tf / roof["peak"], 4)
        del ones_a, ones_b
        # the vendor library on the same A and B, for comparison: torch.mm (hipBLASLt), bf16 out, no C
        # (a lighter job than this GEMM's fp32 D with beta = 1); B transposed into a contiguous copy first
        bt = Bb.t().contiguous()
        for _ in range(3):
            torch.mm(Ab, bt)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(10):
            torch.mm(Ab, bt)
        e1.record(stream)
        e1.synchronize()
        roof["vendor_library"] = {"call": "torch.mm (hipBLASLt): the same bf16 A and B, bf16 D, no C",
                                  "TFLOP/s": round(gemm_flops(M, N, K) / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e12, 1)}
        del bt

    check = None
    if not args.no_check:
        check = spot_check(wb, w8, ws, Db, D8, Ds, Ac, idx, dev)
    del Ab, Bb, Cb, A8, B8, As, Db, D8, Ds, Ac, idx
    torch.cuda.empty_cache()
    configs = None
    if not args.no_configs:
        configs = configs_report(dev, stream, cpu=not args.no_cpu_baseline)
        for p in ("sparse_fp8", "dense_bf16", "dense_fp8", "compress_fp8"):
            configs[{"sparse_fp8": "5s 8192^3 4:2 fp8xbf8 (in the step)", "dense_bf16": "H 8192^3 bf16 beta=1 (in the step)",
                     "dense_fp8": "5d 8192^3 fp8xbf8 (in the step)",
                     "compress_fp8": "5c 8192^2 fp8 4:2 compress (in the step)"}[p]] = report[p]
        configs["5s 8192^3 4:2 fp8xbf8 (in the step)"] = dict(
            report["sparse_fp8"], compress_plus_gemm_ms=round(part_ms["sparse_fp8"] + part_ms["compress_fp8"], 4))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wb, args.cpu_rows)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16,fp8e4m3xbf8e5m2", "data": "synthetic",
        "config": {"workload": "8192^3: 4:2 compress fp8 A + sparse fp8xbf8 GEMM + dense bf16 GEMM "
                               "(beta=1) + dense fp8xbf8 GEMM, fp32 out", "M": M, "N": N, "K": K},
        "parts": report, "roofline": roof, "cpu_baseline": cpu, "check": check, "configs": configs,
        "matrix_rates": rates,
    }
    print(json.dumps(line), flush=True)


def suite():
    """Time each workload on its own: median of repeated launches timed with HIP events on the
    launch stream.  HBM-bound cases rotate through enough copies of their inputs to exceed the
    256 MB Infinity Cache, so they measure HBM, not the cache."""
    import numpy as np
    import torch

    import sparse_matrix_multiply_amd as mm
    import workloads as W

    mm.lib()
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()

    def to_dev(bits, t):
        if t == W.I8:
            return torch.from_numpy(np.ascontiguousarray(bits)).to(dev)
        host = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16 if bits.dtype == np.uint16 else np.int8))
        return host.to(dev).view({W.BF16: torch.bfloat16, W.F16: torch.float16, W.E4M3: torch.float8_e4m3fn,
                                  W.E5M2: torch.float8_e5m2}[t])

    def median_ms(fns, reps):
        """fns: list of callables used round-robin (buffer rotation).  Returns the mean time of one
        launch in a back-to-back batch (throughput; launch overheads overlap) and the median of
        single launches each bracketed by events (latency)."""
        for f in fns[:2]:
            f()
        torch.cuda.synchronize()
        times = []
        for r in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fns[r % len(fns)]()
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for r in range(reps):
            fns[r % len(fns)]()
        e1.record(stream)
        e1.synchronize()
        batch.append(sorted(times)[len(times) // 2])
        return e0.elapsed_time(e1) / reps

    batch = []

    class Progress(dict):
        """The results, with a progress line on stderr as each one comes in (long suite runs under
        a profiler stay visibly alive)."""
        def __setitem__(self, k, v):
            super().__setitem__(k, v)
            print(f"# suite: {k}", file=sys.stderr, flush=True)

    out = Progress()

    def dense_case(name, key, reps=20, rotate=1, n_share=None, bf16_out=False, graph=False):
        """n_share: keep only the first n_share columns of B, C and D (one GPU's share when N is
        split across GPUs).  bf16_out: the epilogue variant with bfloat16 C and D, a per-column
        bias and ReLU."""
        w = dict(W.workload(name))
        if n_share:
            w["B"], w["N"] = w["B"][:n_share], n_share
            if w["C"] is not None:
                w["C"] = np.ascontiguousarray(w["C"][:, :n_share])
        A, B = to_dev(w["A"], w["ta"]), to_dev(w["B"], w["tb"])
        integer = w["ta"] == W.I8
        odt = torch.bfloat16 if bf16_out else torch.int32 if integer else torch.float32
        C = torch.from_numpy(w["C"]).to(dev).to(odt) if w["beta"] != 0 else None
        bias = torch.linspace(-1, 1, w["N"], device=dev) if bf16_out else None
        act = mm.ACT_RELU if bf16_out else mm.ACT_NONE
        Ds = [torch.empty((w["M"], w["N"]), dtype=odt, device=dev) for _ in range(rotate)]
        Bs = [B] + [B.clone() for _ in range(rotate - 1)]
        fns = [lambda s=stream, i=i: mm.gemm_dense(A, Bs[i], Ds[i], w["alpha"], w["beta"], C, a_type=w["ta"],
                                                   b_type=w["tb"], stream=s, bias=bias, act=act)
               for i in range(rotate)]
        ms = median_ms(fns, reps)
        gms = graph_ms(fns, reps) if graph else None
        f = gemm_flops(w["M"], w["N"], w["K"])
        es = 2 if w["ta"] in (W.BF16, W.F16) else 1
        oes = 2 if bf16_out else 4
        byt = (w["M"] + w["N"]) * w["K"] * es + w["M"] * w["N"] * oes * (2 if w["beta"] != 0 else 1)
        out[key] = {"us": round(ms * 1e3, 1), "single_launch_us": round(batch[-1] * 1e3, 1),
                    ("TOP/s" if integer else "TFLOP/s"): round(f / ms / 1e9, 1),
                    "GB/s": round(byt / ms / 1e6, 1), "shape": [w["M"], w["N"], w["K"]], "alpha": w["alpha"],
                    "beta": w["beta"]}
        if gms is not None:
            out[key]["graph_us"] = round(gms * 1e3, 1)
        if bf16_out:
            out[key]["epilogue"] = "bf16 C/D, bias, ReLU"
        del A, B, Bs, C, Ds
        torch.cuda.empty_cache()

    # reference: a plain device copy of the skinny GEMM's bytes, rotated the same way
    n = (16 * 4096 * 2 + 4096 * 4096 * 2 + 2 * 16 * 4096 * 4) // 8
    srcs = [torch.ones(n, dtype=torch.float32, device=dev) for _ in range(16)]
    dsts = [torch.empty_like(x) for x in srcs]
    cms = median_ms([lambda i=i: dsts[i].copy_(srcs[i]) for i in range(16)], 200)
    out["reference_copy_32.6MiB"] = {"us": round(cms * 1e3, 1), "GB/s": round(2 * n * 4 / cms / 1e6, 1)}
    del srcs, dsts
    # and of the 8192^2 fp8 compressor's bytes (64 MiB read, 40 MiB written: 52 MiB copied), 8 copies
    n = (64 + 40) * 2 ** 20 // 2 // 4
    srcs = [torch.ones(n, dtype=torch.float32, device=dev) for _ in range(8)]
    dsts = [torch.empty_like(x) for x in srcs]
    cms = median_ms([lambda i=i: dsts[i].copy_(srcs[i]) for i in range(8)], 80)
    out["reference_copy_52MiB"] = {"us": round(cms * 1e3, 1), "GB/s": round(2 * n * 4 / cms / 1e6, 1)}
    del srcs, dsts

    dense_case("bf16_256", "bf16_256^3", reps=200, graph=True)
    dense_case("i8_1024", "int8_1024^3", reps=200, graph=True)
    dense_case("bf16_4096", "bf16_4096^3_beta1")
    dense_case("bf16_skinny", "bf16_16x4096x4096_beta1", reps=200, rotate=16, graph=True)
    dense_case("bf16_8192", "bf16_8192^3_beta1")
    dense_case("fp8_8192", "fp8e4m3xbf8e5m2_8192^3")
    # one GPU's share of the 8192^3 GEMMs split 8 ways along N
    dense_case("bf16_8192", "share_bf16_8192x1024x8192_beta1", n_share=1024)
    dense_case("fp8_8192", "share_fp8e4m3xbf8e5m2_8192x1024x8192", n_share=1024)

    def split_case(M, N, K, t, key):
        """Small output, long K: unsplit vs the library's split-K plan (synthetic N(0,1) operands)."""
        tdt = {W.BF16: torch.bfloat16, W.E4M3: torch.float8_e4m3fn}[t]
        A = torch.randn(M, K, device=dev).to(tdt)
        B = torch.randn(N, K, device=dev).to(tdt)
        D = torch.empty((M, N), dtype=torch.float32, device=dev)
        ws = mm.workspace(t, M, N, K, device=dev)
        u = median_ms([lambda: mm.gemm_dense(A, B, D, stream=stream)], 50)
        sp = median_ms([lambda: mm.gemm_dense(A, B, D, stream=stream, workspace=ws)], 50)
        f = gemm_flops(M, N, K)
        out[key] = {"unsplit_us": round(u * 1e3, 1), "splitk_us": round(sp * 1e3, 1),
                    "splitk_TFLOP/s": round(f / sp / 1e9, 1), "shape": [M, N, K],
                    "workspace_MiB": round((0 if ws is None else ws.numel()) / 2 ** 20, 1)}
        del A, B, D, ws

    # block-scaled (MX) fp8 x bf8 at 8192^3: E8M0 scales per 32-element block (scale words in the
    # library's k-tile-major layout), 128 x 256 tiles
    w = W.workload("fp8_8192")
    M, N, K = w["M"], w["N"], w["K"]
    A, B = to_dev(w["A"], w["ta"]), to_dev(w["B"], w["tb"])
    SA = torch.full((K // 128, M), 0x7F7F7F7F, dtype=torch.int32, device=dev)
    SB = torch.full((K // 128, N), 0x7F7F7F7F, dtype=torch.int32, device=dev)
    D = torch.empty((M, N), dtype=torch.float32, device=dev)
    ms = median_ms([lambda: mm.gemm_mx(A, SA, B, SB, D, a_type=w["ta"], b_type=w["tb"], stream=stream)], 20)
    out["mx_fp8e4m3xbf8e5m2_8192^3"] = {"us": round(ms * 1e3, 1), "TFLOP/s": round(gemm_flops(M, N, K) / ms / 1e9, 1),
                                         "shape": [M, N, K], "scales": "E8M0 per 32 along K"}
    del A, B, SA, SB, D
    # block-scaled FP4 E2M1 x FP4 at 8192^3 (packed two per byte, random codes)
    g = torch.Generator(device="cpu").manual_seed(5)
    A = torch.randint(0, 256, (M, K // 2), dtype=torch.uint8, generator=g).to(dev)
    B = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, generator=g).to(dev)
    SA = torch.full((K // 128, M), 0x7F7F7F7F, dtype=torch.int32, device=dev)
    SB = torch.full((K // 128, N), 0x7F7F7F7F, dtype=torch.int32, device=dev)
    D = torch.empty((M, N), dtype=torch.float32, device=dev)
    ms = median_ms([lambda: mm.gemm_mx(A, SA, B, SB, D, a_type=mm.FP4_E2M1, b_type=mm.FP4_E2M1, stream=stream)], 20)
    out["mx_fp4e2m1_8192^3"] = {"us": round(ms * 1e3, 1), "TFLOP/s": round(gemm_flops(M, N, K) / ms / 1e9, 1),
                                 "shape": [M, N, K], "scales": "E8M0 per 32 along K"}
    del A, B, SA, SB, D
    # block-scaled FP6 E2M3 x BF6 E3M2 at 8192^3 (packed four per three bytes, random codes)
    A = torch.randint(0, 256, (M, K // 4 * 3), dtype=torch.uint8, generator=g).to(dev)
    B = torch.randint(0, 256, (N, K // 4 * 3), dtype=torch.uint8, generator=g).to(dev)
    SA = torch.full((K // 128, M), 0x7F7F7F7F, dtype=torch.int32, device=dev)
    SB = torch.full((K // 128, N), 0x7F7F7F7F, dtype=torch.int32, device=dev)
    D = torch.empty((M, N), dtype=torch.float32, device=dev)
    ms = median_ms([lambda: mm.gemm_mx(A, SA, B, SB, D, a_type=mm.FP6_E2M3, b_type=mm.BF6_E3M2, stream=stream)], 20)
    out["mx_fp6e2m3xbf6e3m2_8192^3"] = {"us": round(ms * 1e3, 1),
                                         "TFLOP/s": round(gemm_flops(M, N, K) / ms / 1e9, 1),
                                         "shape": [M, N, K], "scales": "E8M0 per 32 along K"}
    del A, B, SA, SB, D

    # other operand layouts: the bf16 8192^3 workload (beta = 1) with A stored M-contiguous and / or
    # B stored N-contiguous (transposed LDS reads)
    w = W.workload("bf16_8192")
    M, N, K = w["M"], w["N"], w["K"]
    A, B = to_dev(w["A"], W.BF16), to_dev(w["B"], W.BF16)
    At, Bt = A.t().contiguous(), B.t().contiguous()
    C = torch.from_numpy(w["C"]).to(dev)
    D = torch.empty((M, N), dtype=torch.float32, device=dev)
    for ta, tb, key in ((True, False, "A_Mcontig"), (False, True, "B_Ncontig"), (True, True, "A_Mcontig_B_Ncontig")):
        ms = median_ms([lambda: mm.gemm_layout(At if ta else A, Bt if tb else B, D, ta, tb, 1.0, 1.0, C,
                                               stream=stream)], 20)
        out["layout_bf16_8192^3_beta1_" + key] = {"us": round(ms * 1e3, 1),
                                                  "TFLOP/s": round(gemm_flops(M, N, K) / ms / 1e9, 1)}
    del A, B, At, Bt, C, D
    # the same for the 8192^3 fp8 x bf8 workload (transposed 8-bit reads)
    w = W.workload("fp8_8192")
    A, B = to_dev(w["A"], w["ta"]), to_dev(w["B"], w["tb"])
    At, Bt = A.t().contiguous(), B.t().contiguous()
    D = torch.empty((M, N), dtype=torch.float32, device=dev)
    for ta, tb, key in ((True, False, "A_Mcontig"), (False, True, "B_Ncontig"), (True, True, "A_Mcontig_B_Ncontig")):
        ms = median_ms([lambda: mm.gemm_layout(At if ta else A, Bt if tb else B, D, ta, tb, a_type=w["ta"],
                                               b_type=w["tb"], stream=stream)], 20)
        out["layout_fp8e4m3xbf8e5m2_8192^3_" + key] = {"us": round(ms * 1e3, 1),
                                                       "TFLOP/s": round(gemm_flops(M, N, K) / ms / 1e9, 1)}
    del A, B, At, Bt, D
    torch.cuda.empty_cache()

    split_case(512, 512, 32768, W.BF16, "splitk_bf16_512x512x32768")
    split_case(256, 256, 65536, W.BF16, "splitk_bf16_256x256x65536")
    split_case(1024, 512, 8192, W.E4M3, "splitk_fp8e4m3_1024x512x8192")
    # epilogue variant: bfloat16 C and D with bias and ReLU (half the output bytes)
    dense_case("bf16_8192", "bf16_8192^3_beta1_bf16out_bias_relu", bf16_out=True)
    dense_case("fp8_8192", "fp8e4m3xbf8e5m2_8192^3_bf16out_bias_relu", bf16_out=True)
    dense_case("bf16_skinny", "bf16_16x4096x4096_beta1_bf16out_bias_relu", reps=200, rotate=16, bf16_out=True)

    for name, key, rot, n_share in (("f16_sparse", "f16_4:2_4096x4096x8192", 8, None),
                                    ("fp8_8192_sparse", "fp8_4:2_8192^3", 8, None),
                                    ("fp8_8192_sparse", "share_fp8_4:2_8192x1024x8192", 8, 1024)):
        w = dict(W.workload(name))
        if n_share:
            w["B"], w["N"] = w["B"][:n_share], n_share
        ta, tb, M, N, K = w["ta"], w["tb"], w["M"], w["N"], w["K"]
        As = [to_dev(w["A"], ta)]
        As += [As[0].clone() for _ in range(rot - 1)]
        tdt = As[0].dtype
        Acs = [torch.empty((M, K // 2), dtype=tdt, device=dev) for _ in range(rot)]
        idxs = [torch.empty((M, K // 32), dtype=torch.int32, device=dev) for _ in range(rot)]
        cms = median_ms([lambda i=i: mm.sparse24_compress(As[i], Acs[i], idxs[i], a_type=ta, stream=stream)
                         for i in range(rot)], 40)
        pms = median_ms([lambda i=i: mm.sparse24_prune_compress(As[i], Acs[i], idxs[i], a_type=ta, stream=stream)
                         for i in range(rot)], 40)
        es = 2 if ta in (W.BF16, W.F16) else 1
        cbytes = M * K * es + M * (K // 2) * es + M * (K // 32) * 4
        B = to_dev(w["B"], tb)
        D = torch.empty((M, N), dtype=torch.float32, device=dev)
        gms = median_ms([lambda: mm.gemm_sparse24(Acs[0], idxs[0], B, D, K=K, a_type=ta, b_type=tb, stream=stream)], 20)
        f = gemm_flops(M, N, K)

        out[key] = {"compress_us": round(cms * 1e3, 1), "compress_GB/s": round(cbytes / cms / 1e6, 1),
                    "prune_compress_us": round(pms * 1e3, 1), "prune_compress_GB/s": round(cbytes / pms / 1e6, 1),
                    "gemm_us": round(gms * 1e3, 1), "TFLOP/s_dense_equivalent": round(f / gms / 1e9, 1),
                    "TFLOP/s_effective": round(f / 2 / gms / 1e9, 1), "shape": [M, N, K]}

        del As, Acs, idxs, B, D
        torch.cuda.empty_cache()
    print(json.dumps({"suite": out, "note": "us: mean of back-to-back launches issued from Python (HIP events on "
                      "the launch stream); single_launch_us: median of single launches, each between events; "
                      "graph_us: back-to-back launches replayed from a HIP graph (no host cost per call); the "
                      "skinny GEMM and the compressors rotate through copies larger than the 256 MB Infinity "
                      "Cache"}), flush=True)


def only(which, steps, warmup):
    """One kernel by itself, for counter runs: mean time per launch of `steps` back-to-back launches
    after `warmup` (HIP events on the launch stream), as one JSON line."""
    import numpy as np
    import torch

    import sparse_matrix_multiply_amd as mm
    import workloads as W
    mm.lib()
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    if which == "rates":
        print(json.dumps({"only": which, "matrix_rates": matrix_rates()}), flush=True)
        return

    def to_dev(bits, t):
        host = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16 if bits.dtype == np.uint16 else np.int8))
        return host.to(dev).view({W.BF16: torch.bfloat16, W.E4M3: torch.float8_e4m3fn}[t])

    if which in ("bf16_8192", "bf16_8192_ones"):
        # the step's bf16 GEMM (beta = 1) alone, on its random inputs or on all-ones A and B
        w = W.workload("bf16_8192")
        M, N, K = w["M"], w["N"], w["K"]
        if which == "bf16_8192":
            A, B = to_dev(w["A"], W.BF16), to_dev(w["B"], W.BF16)
        else:
            A = torch.ones((M, K), dtype=torch.bfloat16, device=dev)
            B = torch.ones((N, K), dtype=torch.bfloat16, device=dev)
        C = torch.from_numpy(w["C"]).to(dev)
        D = torch.empty((M, N), dtype=torch.float32, device=dev)
        fns = [lambda: mm.gemm_dense(A, B, D, 1.0, 1.0, C, stream=stream)]
        nbytes = (M + N) * K * 2 + 2 * M * N * 4
    elif which == "skinny":
        w = W.workload("bf16_skinny")
        M, N, K = w["M"], w["N"], w["K"]
        A = to_dev(w["A"], W.BF16)
        Bs = [to_dev(w["B"], W.BF16)]
        Bs += [Bs[0].clone() for _ in range(15)]
        C = torch.from_numpy(w["C"]).to(dev)
        Ds = [torch.empty((M, N), dtype=torch.float32, device=dev) for _ in range(16)]
        fns = [lambda i=i: mm.gemm_dense(A, Bs[i], Ds[i], 1.0, 1.0, C, stream=stream) for i in range(16)]
        nbytes = (M + N) * K * 2 + 2 * M * N * 4
    else:
        w = W.workload("fp8_8192_sparse")
        M, K = w["M"], w["K"]
        As = [to_dev(w["A"], W.E4M3)]
        As += [As[0].clone() for _ in range(7)]
        Acs = [torch.empty((M, K // 2), dtype=torch.float8_e4m3fn, device=dev) for _ in range(8)]
        idxs = [torch.empty((M, K // 32), dtype=torch.int32, device=dev) for _ in range(8)]
        fns = [lambda i=i: mm.sparse24_compress(As[i], Acs[i], idxs[i], a_type=W.E4M3, stream=stream) for i in range(8)]
        nbytes = M * K + M * (K // 2) + M * (K // 32) * 4
    for r in range(warmup):
        fns[r % len(fns)]()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for r in range(steps):
        fns[r % len(fns)]()
    e1.record(stream)
    e1.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    out = {"only": which, "launches": steps, "us": round(us, 2), "algorithmic_bytes": nbytes,
           "GB/s": round(nbytes / us / 1e3, 1)}
    if which.startswith("bf16_8192"):
        out["TFLOP/s"] = round(gemm_flops(M, N, K) / us / 1e6, 1)
    print(json.dumps(out), flush=True)


def matrix_rates():
    """Sustained rate of the matrix instructions the GEMM kernels use, each issued back to back on
    every compute unit for about 150 ms (libmmac_rate.so), once on constant operands and once on
    random ones that change from one instruction to the next (as a GEMM's fragments do), with the
    shader clock each run holds: the ceiling this GPU reaches, beside the published peaks."""
    from sparse_matrix_multiply_amd import rate
    out = {}
    for key, instr, peak in (("bf16_mfma", rate.MFMA_BF16, PEAK_TFLOPS["bf16"]), ("fp8_mfma", rate.MFMA_FP8, PEAK_TFLOPS["fp8"]),
                             ("i8_mfma", rate.MFMA_I8, PEAK_TFLOPS["int8"]),
                             ("fp16_smfmac", rate.SMFMAC_F16, 2 * PEAK_TFLOPS["fp16"]),
                             ("fp8_smfmac", rate.SMFMAC_FP8, 2 * PEAK_TFLOPS["fp8"]),
                             ("fp6_mfma_scaled", rate.MFMA_FP6, PEAK_TFLOPS["fp6"]),
                             ("fp4_mfma_scaled", rate.MFMA_FP4, PEAK_TFLOPS["fp4"])):
        out[key] = {"instr": rate.name(instr)}
        for kind, rnd in (("constant_operands", False), ("random_operands", True)):
            r = rate.measure(instr, random=rnd)
            out[key][kind] = {"TFLOP/s": round(r["TFLOP/s"], 1), "frac_published": round(r["TFLOP/s"] / peak, 4),
                              "sclk_MHz": round(r["sclk_GHz"] * 1000), "cycles_per_instr": round(r["cycles_per_instr"], 2),
                              "seconds": round(r["seconds"], 3)}
    return out


def graph_ms(fns, reps):
    """Mean time of one launch when `reps` calls (the fns round-robin; each takes the stream to launch
    on) are captured in one HIP graph and the graph is replayed: the GPU's back-to-back time without
    the host's cost per call, which for a small GEMM is as long as the kernel itself.  Median of
    three timed replays after one untimed one."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream()
        for r in range(reps):
            fns[r % len(fns)](cap)
    times = []
    for _ in range(4):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1) / reps)
    del g
    return sorted(times[1:])[1]


def configs_report(dev, stream, cpu=True):
    """The smaller workloads at their full sizes: GPU time per launch of back-to-back launches, timed
    two ways ("us_graph": replayed from a HIP graph; "us_eager": issued one by one from Python, which
    for the smallest kernels takes longer than the kernel; HIP events on the launch stream; "us" is
    the lower; "us_single_median" / "us_single_min": launches one at a time, each between its own
    events; the HBM-bound ones rotate through copies larger than the 256 MB Infinity Cache, and
    "us_warm" repeats one copy, resident in that cache), a full comparison with the oracle, and the
    oracle's own wall time on the host's cores (the 256^3 and 1024^3 int8 workloads also on one
    thread)."""
    import numpy as np
    import torch

    import oracle
    import sparse_matrix_multiply_amd as mm
    import workloads as W

    threads = oracle.num_threads()
    U = 2.0 ** -24

    def to_dev(bits, t):
        if t == W.I8:
            return torch.from_numpy(np.ascontiguousarray(bits)).to(dev)
        host = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16 if bits.dtype == np.uint16 else np.int8))
        return host.to(dev).view({W.BF16: torch.bfloat16, W.F16: torch.float16, W.E4M3: torch.float8_e4m3fn,
                                  W.E5M2: torch.float8_e5m2}[t])

    def mean_ms(fns, reps):
        for f in fns[:2]:
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for r in range(reps):
            fns[r % len(fns)]()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / reps

    def single_ms(fns, reps):
        """(median, min) of single launches, each between its own pair of HIP events."""
        times = []
        for r in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fns[r % len(fns)]()
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        times.sort()
        return times[len(times) // 2], times[0]

    def timed_oracle(fn, one_thread=False):
        if not cpu:
            return None, None
        t = time.perf_counter()
        res = fn()
        out = {"seconds": round(time.perf_counter() - t, 3), "threads": threads}
        if one_thread:
            oracle.set_num_threads(1)
            t = time.perf_counter()
            fn()
            out["seconds_1_thread"] = round(time.perf_counter() - t, 3)
            oracle.set_num_threads(threads)
        return res, out

    def gate(D, ref, S, K, alpha, beta, C):
        """normwise and element-wise errors of the float gates (the parity tests' bound; no narrow
        format here), and whether both pass."""
        D, ref = np.asarray(D, np.float64), np.asarray(ref, np.float64)
        scale = abs(alpha) * S + (abs(beta) * np.abs(C.astype(np.float64)) if beta != 0 else 0.0)
        e = oracle.normwise_error(D, ref, S, alpha, beta, C if beta != 0 else None)
        emax = float(np.max(np.abs(D - ref) / np.where(scale > 0, scale, 1.0)))
        ok = e <= 8 * U * np.sqrt(K) and emax <= 2 * (K + 2) * U
        return {"normwise": float(f"{e:.3e}"), "elementwise": float(f"{emax:.3e}"), "pass": bool(ok)}

    out = {}
    if cpu:
        oracle.lib()
    for name, key, reps, rot in (("bf16_256", "1 bf16 256^3", 200, 1), ("i8_1024", "2 int8 1024^3", 200, 1),
                                 ("bf16_4096", "3a bf16 4096^3 beta=1", 20, 1),
                                 ("bf16_skinny", "3b bf16 16x4096x4096 beta=1", 200, 16)):
        w = W.workload(name)
        M, N, K, ta = w["M"], w["N"], w["K"], w["ta"]
        integer = ta == W.I8
        A = to_dev(w["A"], ta)
        Bs = [to_dev(w["B"], w["tb"])]
        Bs += [Bs[0].clone() for _ in range(rot - 1)]
        odt = torch.int32 if integer else torch.float32
        C = torch.from_numpy(w["C"]).to(dev) if w["beta"] != 0 else None
        Ds = [torch.empty((M, N), dtype=odt, device=dev) for _ in range(rot)]
        fns = [lambda s=stream, i=i: mm.gemm_dense(A, Bs[i], Ds[i], w["alpha"], w["beta"], C, a_type=ta,
                                                   b_type=w["tb"], stream=s) for i in range(rot)]
        eager = mean_ms(fns, reps)
        torch.cuda.synchronize()
        D = Ds[0].cpu().numpy()
        graph = graph_ms(fns, reps)
        replay_same = bool(np.array_equal(Ds[0].cpu().numpy(), D))
        ms = min(graph, eager)
        byt = (M + N) * K * (2 if ta == W.BF16 else 1) + M * N * 4 * (2 if w["beta"] != 0 else 1)
        med, mn = single_ms(fns, reps)
        r = {"shape": [M, N, K], "us": round(ms * 1e3, 2), "us_graph": round(graph * 1e3, 2),
             "us_eager": round(eager * 1e3, 2), "us_single_median": round(med * 1e3, 2),
             "us_single_min": round(mn * 1e3, 2),
             ("TOP/s" if integer else "TFLOP/s"): round(gemm_flops(M, N, K) / ms / 1e9, 1),
             "GB/s": round(byt / ms / 1e6, 1), "graph_replay_matches_eager": replay_same}
        if rot > 1:
            # the same launches without rotation: B stays resident in the 256 MB Infinity Cache
            r["rotated_copies"] = rot
            warm = mean_ms(fns[:1], reps)
            r["us_warm"] = round(warm * 1e3, 2)
            r["GB/s_warm"] = round(byt / warm / 1e6, 1)
        res, r["oracle"] = timed_oracle(lambda: oracle.gemm_dense(ta, w["tb"], w["A"], w["B"], w["alpha"], w["beta"], w["C"]),
                                        one_thread=name in ("bf16_256", "i8_1024"))
        if res is not None:
            ref, aux = res
            r["check"] = {"bit_exact": bool(np.array_equal(D, ref))} if integer else gate(D, ref, aux, K, w["alpha"], w["beta"], w["C"])
        out[key] = r
        del A, Bs, C, Ds
        torch.cuda.empty_cache()

    # the floor under the small cases: a one-element fill (torch's, the least a kernel can do) and the
    # library's smallest GEMM (64 x 64 x 64 bf16, one k-tile: prologue, one step, epilogue), replayed
    # from a HIP graph like the small cases above
    one = torch.zeros(1, device=dev)
    a64 = torch.zeros((64, 64), dtype=torch.bfloat16, device=dev)
    d64 = torch.empty((64, 64), dtype=torch.float32, device=dev)
    out["launch_floor"] = {
        "us_graph_one_element_fill": round(graph_ms([lambda s: one.fill_(0.0)], 200) * 1e3, 2),
        "us_graph_gemm_64x64x64_bf16": round(graph_ms([lambda s: mm.gemm_dense(a64, a64, d64, stream=s)], 200) * 1e3, 2)}
    del one, a64, d64

    # 4:2 fp16 4096 x 4096 x 8192: compression of the dense A (rotated), then the sparse GEMM
    w = W.workload("f16_sparse")
    M, N, K, ta = w["M"], w["N"], w["K"], w["ta"]
    As = [to_dev(w["A"], ta)]
    As += [As[0].clone() for _ in range(7)]
    Acs = [torch.empty((M, K // 2), dtype=torch.float16, device=dev) for _ in range(8)]
    idxs = [torch.empty((M, K // 32), dtype=torch.int32, device=dev) for _ in range(8)]
    cfns = [lambda i=i: mm.sparse24_compress(As[i], Acs[i], idxs[i], a_type=ta, stream=stream) for i in range(8)]
    cms = mean_ms(cfns, 40)
    cwarm = mean_ms(cfns[:1], 40)
    B = to_dev(w["B"], w["tb"])
    D = torch.empty((M, N), dtype=torch.float32, device=dev)
    gms = mean_ms([lambda: mm.gemm_sparse24(Acs[0], idxs[0], B, D, K=K, a_type=ta, b_type=w["tb"], stream=stream)], 20)
    torch.cuda.synchronize()
    cbytes = M * K * 2 + M * (K // 2) * 2 + M * (K // 32) * 4
    r = {"shape": [M, N, K], "compress_us": round(cms * 1e3, 2), "compress_GB/s": round(cbytes / cms / 1e6, 1),
         "compress_us_warm": round(cwarm * 1e3, 2), "compress_GB/s_warm": round(cbytes / cwarm / 1e6, 1),
         "gemm_us": round(gms * 1e3, 2), "TFLOP/s_dense_equivalent": round(gemm_flops(M, N, K) / gms / 1e9, 1),
         "TFLOP/s_effective": round(gemm_flops(M, N, K) / 2 / gms / 1e9, 1),
         "compress_plus_gemm_us": round((cms + gms) * 1e3, 2)}
    Acg = Acs[0].view(torch.int16).cpu().numpy().view(np.uint16)
    idxg = idxs[0].cpu().numpy().view(np.uint32)
    Dg = D.cpu().numpy()
    res, r["oracle_compress"] = timed_oracle(lambda: oracle.compress24(ta, w["A"]))
    if res is not None:
        Ac_ref, idx_ref, _ = res
        r["check_compress"] = {"bit_exact": bool(np.array_equal(Acg, Ac_ref) and np.array_equal(idxg, idx_ref))}
        res, r["oracle"] = timed_oracle(lambda: oracle.gemm_sparse24(ta, w["tb"], Ac_ref, idx_ref, w["B"]))
        ref, S = res
        r["check"] = gate(Dg, ref, S, K, 1.0, 0.0, None)
    out["4 fp16 4:2 4096x4096x8192"] = r
    del As, Acs, idxs, B, D
    torch.cuda.empty_cache()
    return out


def spot_check(wb, w8, ws, Db, D8, Ds, Ac, idx, dev):
    """Compare 512 sampled outputs of each GEMM (and the index words) with the oracle."""
    import numpy as np
    import torch
    import oracle

    g = np.random.default_rng(1)
    ii = g.integers(0, 8192, 512)
    jj = g.integers(0, 8192, 512)
    it, jt = torch.from_numpy(ii).to(dev), torch.from_numpy(jj).to(dev)
    out = {}
    for name, w, D in (("dense_bf16", wb, Db), ("dense_fp8", w8, D8)):
        ref, S = oracle.gemm_dense_entries(w["ta"], w["tb"], w["A"], w["B"], ii, jj, w["alpha"], w["beta"], w["C"])
        C = w["C"][ii, jj] if w["beta"] != 0 else None
        e = oracle.normwise_error(D[it, jt].cpu().numpy(), ref, S, w["alpha"], w["beta"], C)
        out[name] = float(f"{e:.3e}")
    Ac_ref, idx_ref, _ = oracle.compress24(ws["ta"], ws["A"])
    out["index_words_match"] = bool(np.array_equal(idx.cpu().numpy().view(np.uint32), idx_ref))
    out["compressed_values_match"] = bool(np.array_equal(
        Ac.view(torch.int8).cpu().numpy().view(np.uint8), Ac_ref))
    ref, S = oracle.gemm_sparse24_entries(ws["ta"], ws["tb"], Ac_ref, idx_ref, ws["B"], ii, jj)
    e = oracle.normwise_error(Ds[it, jt].cpu().numpy(), ref, S, 1.0, 0.0)
    out["sparse_fp8"] = float(f"{e:.3e}")
    return out


def cpu_baseline(wb, rows):
    """Time the oracle on a slice of the bf16 8192^3 GEMM's output rows (all 8192 columns)."""
    import oracle
    threads = oracle.num_threads()
    if rows <= 0:
        # calibrate to about 15 s of CPU work: two probes, so the fixed cost (decoding B) cancels
        def timed(r):
            t = time.perf_counter()
            oracle.gemm_dense(wb["ta"], wb["tb"], wb["A"], wb["B"], wb["alpha"], wb["beta"], wb["C"], rows=(0, r))
            return time.perf_counter() - t
        r1, r2 = threads, 3 * threads
        per_row = max((timed(r2) - timed(r1)) / (r2 - r1), 1e-4)
        rows = int(min(8192, max(threads, 15.0 / per_row)))
    t = time.perf_counter()
    oracle.gemm_dense(wb["ta"], wb["tb"], wb["A"], wb["B"], wb["alpha"], wb["beta"], wb["C"], rows=(0, rows))
    dt = time.perf_counter() - t
    return {"value": round(gemm_flops(rows, 8192, 8192) / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"bf16 GEMM, output rows 0..{rows - 1} of 8192x8192x8192 (fp64 accumulation), {dt:.1f} s"}


if __name__ == "__main__":
    main()
