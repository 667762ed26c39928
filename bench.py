"""Benchmark of the MI355X blocked GEMM on one GPU; prints one JSON line.

A step is one C = A.B call through the C ABI on the headline workload (default:
the square bf16 product 8192 x 8192 x 8192, A row-major, B column-major, f16
output), inputs already resident in HBM.  Timing: W untimed warm-up steps, then
K steps between two device synchronisations, measured with HIP events on the
stream the kernels are launched on (torch's current stream).  As a second
estimate, the median over 7 interleaved trials of (t(n2) - t(n1)) / (n2 - n1) is
reported, which removes fixed launch overheads.

Also reported:
  roofline      achieved algorithmic TFLOP/s (or GB/s) of the GEMM kernel against
                the MI355X peak, plus HBM traffic from committed rocprofv3 counter
                summaries when they belong to the current kernel source;
  cpu_baseline  the CPU oracle timed on a bounded sample of the same workload
                (whole output rows), on all host threads it uses;
  secondary     the skinny batched workload (16 x 16384 x 8192, batch 8) in
                GB/s against HBM peak, unless --no-secondary.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_PEAK_TFLOPS = 2516.6   # dense f16/bf16: 256 CUs x 4096 FLOP/clk x 2.4 GHz
HBM_PEAK_GBS = 8000.0       # HBM3E
METRIC = "GEMM TFLOP/s + % of MI355X fp16 MFMA peak (HBM GB/s for skinny M)"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tiled_shared_memory_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload, kernel):
    """HBM bytes per launch from a committed counter summary of the same kernel source, else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash() or rec.get("kernel") != kernel:
        return None
    return rec.get("hbm_bytes_per_launch")


class Setup:
    """Inputs of one workload uploaded to the GPU, and a closure that runs one step."""

    def __init__(self, w, torch, tsm):
        self.w = w
        log(f"generating {w.name} inputs on the host")
        t0 = time.time()
        self.A, self.B = w.operands()
        log(f"generated in {time.time() - t0:.1f} s; uploading")
        import numpy as np

        self.a = torch.from_numpy(self.A.reshape(-1).view(np.int16)).cuda()
        self.b = torch.from_numpy(self.B.reshape(-1).view(np.int16)).cuda()
        out_dt = torch.float32 if w.out_fmt == "f32" else torch.float16
        self.c = torch.empty(w.batch * w.M * w.N, dtype=out_dt, device="cuda")
        self.lda, self.ldb, self.ldc = w.lds()
        self.sA, self.sB, self.sC = w.strides()
        self.code = {("f16", "f32"): tsm.TSM_F16_F32, ("f16", "f16"): tsm.TSM_F16_F16,
                     ("bf16", "f32"): tsm.TSM_BF16_F32, ("bf16", "f16"): tsm.TSM_BF16_F16}[(w.in_fmt, w.out_fmt)]
        self.la = tsm.TSM_COL if w.a_layout == "col" else tsm.TSM_ROW
        self.lb = tsm.TSM_COL if w.b_layout == "col" else tsm.TSM_ROW
        self.stream = torch.cuda.current_stream()
        self.handle = self.stream.cuda_stream
        self.tsm = tsm
        self.torch = torch
        self.args = (w.M, w.N, w.K, self.a, self.lda, self.la, self.sA, self.b, self.ldb, self.lb, self.sB, self.c,
                     self.ldc, self.sC, w.batch, self.code)
        self.kernel = tsm.tsm_gemm_kernel_name(*self.args)

    def step(self):
        self.tsm.gemm_strided_batched_ex(*self.args, self.handle)

    def time_steps(self, n):
        torch = self.torch
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(self.stream)
        for _ in range(n):
            self.step()
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def interleaved_ms(self, n1=2, n2=12, trials=7):
        vals = []
        for _ in range(trials):
            t1 = self.time_steps(n1)
            t2 = self.time_steps(n2)
            vals.append((t2 - t1) / (n2 - n1))
        return statistics.median(vals)

    def check_cells(self, orc, ncells=64):
        """Sampled parity of the benchmarked output against the oracle."""
        import numpy as np

        import oracle

        w = self.w
        self.torch.cuda.synchronize()
        rng = np.random.default_rng(2024)
        z = rng.integers(0, w.batch, ncells)
        i = rng.integers(0, w.M, ncells)
        j = rng.integers(0, w.N, ncells)
        host = self.c.cpu().numpy().astype(np.float64).reshape(w.batch, w.M, w.N)
        got = host[z, i, j]
        ref, S = orc.gemm_points(self.A, self.B, w.M, w.N, w.K, w.in_fmt, z, i, j, strideA=self.A[0].size,
                                 strideB=self.B[0].size, a_layout=w.a_layout, b_layout=w.b_layout)
        bnd = oracle.bound(w.K, S, w.out_fmt, got)
        ratio = float(np.max(np.abs(got - ref) / np.where(bnd > 0, bnd, 1.0)))
        return {"cells": ncells, "max_err_over_bound": ratio, "pass": bool(ratio <= 1.0 and np.all(np.isfinite(got)))}


def cpu_baseline(orc, w, A, B, target_s):
    """Oracle timed on whole output rows of problem 0; rows chosen for about target_s seconds.

    Two short runs fit t(rows) = fixed + per_row * rows (the fixed part decodes
    B); the timed run then takes about target_s seconds.
    """
    def run(rows):
        t0 = time.perf_counter()
        orc.gemm_rows(A[:1], B[:1], w.M, w.N, w.K, w.in_fmt, a_layout=w.a_layout, b_layout=w.b_layout,
                      row_begin=0, row_end=rows)
        return time.perf_counter() - t0

    r1, r2 = min(w.M, 16), min(w.M, 64)
    t1, t2 = run(r1), run(r2)
    per_row = max((t2 - t1) / max(r2 - r1, 1), 1e-6)
    fixed = max(t1 - per_row * r1, 0.0)
    rows = max(1, min(w.M, int((target_s - fixed) / per_row)))
    t = run(rows)
    flops = 2.0 * rows * w.N * w.K
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": orc.threads(), "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of problem 0 ({rows} x {w.N} x {w.K} fp64 multiply-adds, "
                      f"{t:.1f} s including the decode of B)",
            "seconds": t}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="square_bf16_8192")
    ap.add_argument("--secondary", default="skinny_f16_16x16384x8192_b8")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (to scale HBM counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the data-parallel sharding across GPUs is described in DESIGN.md, not built)", file=sys.stderr)
        sys.exit(2)

    import torch

    import tiled_shared_memory_amd as tsm
    from workloads import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 2
        src = torch.ones(n, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": 2 * n}), flush=True)
        return
    tsm.load()
    w = WORKLOADS[args.workload]
    s = Setup(w, torch, tsm)
    log(f"kernel {s.kernel}; warm-up {args.warmup}")
    for _ in range(args.warmup):
        s.step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    total_ms = s.time_steps(args.steps)
    ms = total_ms / args.steps
    ms_interleaved = s.interleaved_ms()
    log(f"{ms:.4f} ms/step (interleaved median {ms_interleaved:.4f} ms)")

    import oracle

    orc = oracle.default()
    check = s.check_cells(orc)
    tflops = w.flops / (ms * 1e-3) / 1e12
    gbs = w.bytes / (ms * 1e-3) / 1e9
    compute_bound = w.flops / w.bytes > MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    traffic = traffic_from_profiles(w.name, s.kernel)
    if compute_bound:
        roof = {"bound": "mfma", "achieved": tflops, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": tflops / MFMA_PEAK_TFLOPS, "traffic": traffic}
    else:
        roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gbs / HBM_PEAK_GBS, "traffic": traffic}
    roof["kernel"] = s.kernel
    roof["algorithmic_flops_per_launch"] = w.flops
    roof["algorithmic_bytes_per_launch"] = w.bytes

    result = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.in_fmt,
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "batch": w.batch, "in": w.in_fmt,
                   "out": w.out_fmt, "a_layout": w.a_layout, "b_layout": w.b_layout, "seed": w.seed,
                   "parallelism": "single GPU", "accumulate": "f32"},
        "pct_of_mfma_peak": 100.0 * tflops / MFMA_PEAK_TFLOPS,
        "hbm_gbs_algorithmic": gbs,
        "ms_per_step_interleaved_median": ms_interleaved,
        "check": check,
        "roofline": roof,
    }
    # free the headline operands before the secondary workload
    s_main = s
    del s

    if not args.no_secondary and args.secondary:
        w2 = WORKLOADS[args.secondary]
        s2 = Setup(w2, torch, tsm)
        for _ in range(max(3, args.warmup // 2)):
            s2.step()
        torch.cuda.synchronize()
        n2 = max(10, args.steps // 2)
        ms2 = s2.time_steps(n2) / n2
        ms2i = s2.interleaved_ms()
        check2 = s2.check_cells(orc)
        gbs2 = w2.bytes / (ms2 * 1e-3) / 1e9
        result["secondary"] = {
            "workload": w2.name, "kernel": s2.kernel, "ms_per_step": ms2, "ms_per_step_interleaved_median": ms2i,
            "hbm_gbs_algorithmic": gbs2, "pct_of_hbm_peak": 100.0 * gbs2 / HBM_PEAK_GBS,
            "tflops": w2.flops / (ms2 * 1e-3) / 1e12, "check": check2,
            "roofline": {"bound": "hbm", "achieved": gbs2, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs2 / HBM_PEAK_GBS, "traffic": traffic_from_profiles(w2.name, s2.kernel)},
        }
        log(f"secondary {w2.name}: {ms2:.4f} ms, {gbs2:.0f} GB/s")
        del s2

    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(orc, w, s_main.A, s_main.B, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
