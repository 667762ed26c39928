"""Benchmark of the MI355X blocked GEMM on one GPU; prints one JSON line.

A step is one C = A.B call through the C ABI on the headline workload (default:
the square bf16 product 8192 x 8192 x 8192, A row-major, B column-major, f16
output), inputs already resident in HBM.  Timing: the step runs untimed for at
least --settle seconds (the GPU leaves its idle clock only after some tens of
milliseconds of load: the first 10 steps after an idle gap average 0.87 ms,
steps 40-50 0.74 ms, the settled rate 0.73 ms), then W untimed warm-up steps,
then K steps between two device synchronisations, measured with HIP events on
the stream the kernels are launched on (torch's current stream).  Before any
timing, one step writes C over a NaN fill and every element is checked finite
on the GPU.  As a second estimate, the median over 7 interleaved trials of
(t(n2) - t(n1)) / (n2 - n1) is reported, which removes fixed launch overheads.

Also reported:
  roofline      achieved algorithmic TFLOP/s (or GB/s) of the GEMM kernel against
                the MI355X peak, plus HBM traffic from committed rocprofv3 counter
                summaries when they belong to the current kernel source;
  cpu_baseline  the CPU oracle timed on the same workload (the whole product
                when it takes under --cpu-max-seconds, else whole output rows),
                on all host threads it uses;
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


# Sources that define each kernel family's device code (with the shared headers
# below): a counter record stays valid while these are unchanged.
KERNEL_FILES = {"tile_": ("gemm_tile.hip",), "skinny_": ("gemm_skinny.hip",),
                "hybrid_": ("gemm_tile.hip", "gemm_ksplit.hip"), "streamk_": ("gemm_tile.hip", "gemm_ksplit.hip"),
                "band_": ("gemm_tile.hip", "gemm_masked.hip", "gemm_skinny.hip", "gemm_splitk.hip"),
                "ksplit_": ("gemm_skinny.hip", "gemm_ksplit.hip", "gemm_tile.hip"),
                "splitk_": ("gemm_splitk.hip",), "masked_": ("gemm_masked.hip",), "rowsum_": ("rowsum.hip",)}
SHARED_FILES = ("gemm_internal.hpp", "mfma.hpp")


def kernel_source_hash(kernel=None):
    """Hash of the kernel sources: of every file under csrc/, or, given a kernel name, of its family's files."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tiled_shared_memory_amd", "csrc")
    if kernel is None:
        files = [f for f in sorted(os.listdir(csrc)) if f.endswith((".hip", ".hpp", ".h"))]
    else:
        fam = next(v for k, v in KERNEL_FILES.items() if kernel.startswith(k))
        files = sorted(set(fam) | set(SHARED_FILES))
    for f in files:
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
    if rec.get("source_hash") != kernel_source_hash(kernel) or rec.get("kernel") != kernel:
        return None
    return rec.get("hbm_bytes_per_launch")


# The measurement run that --summarize reads: each command's output directory
# under RUN_DIR, and the command (run from /tmp, with TMPDIR=/tmp).
# WORKLOAD_ARGS stands for the run's workload flags (none for the default run).
PROFILE_COMMANDS = {
    "bench.json": "python3 bench.py WORKLOAD_ARGS > RUN_DIR/bench.json",
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d RUN_DIR/trace -o bench -- "
             "python3 bench.py WORKLOAD_ARGS --no-cpu-baseline",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d RUN_DIR/fetch -o p -- "
             "python3 bench.py WORKLOAD_ARGS --no-cpu-baseline --settle 0 --steps 5 --warmup 2",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d RUN_DIR/write -o p -- "
             "python3 bench.py WORKLOAD_ARGS --no-cpu-baseline --settle 0 --steps 5 --warmup 2",
    "cal_fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d RUN_DIR/cal_fetch -o c -- "
                 "python3 bench.py --calibrate-copy 1024",
    "cal_write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d RUN_DIR/cal_write -o c -- "
                 "python3 bench.py --calibrate-copy 1024",
    "sq": "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS "
          "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F16 GRBM_GUI_ACTIVE --output-format csv "
          "-d RUN_DIR/sq -o p -- python3 bench.py WORKLOAD_ARGS --no-cpu-baseline --settle 0 --steps 5 --warmup 2",
}
# Where the MFMA pipes lose cycles: the same passes on the headline kernel (KERNEL_ARGS: none) and on
# torch.matmul (KERNEL_ARGS: --torch-reference), one pass per counter group.
STALL_PASSES = {
    "waits": "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_VALU_MFMA_BUSY_CYCLES "
             "SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_VMEM GRBM_GUI_ACTIVE",
    "vmem_latency": "VmemLatency",
    "lds_latency": "LdsLatency",
    "fifo": "SQ_WAIT_INST_LDS SQ_LDS_DATA_FIFO_FULL SQ_LDS_CMD_FIFO_FULL SQ_VMEM_TA_ADDR_FIFO_FULL "
            "SQ_VMEM_TA_CMD_FIFO_FULL SQ_ACTIVE_INST_SCA SQ_ACTIVE_INST_MISC SQ_INSTS_SALU GRBM_GUI_ACTIVE",
    "l1": "TA_TA_BUSY TA_ADDR_STALLED_BY_TC_CYCLES TCP_TCC_READ_REQ_LATENCY TCP_TCC_READ_REQ "
          "TCP_PENDING_STALL_CYCLES TCP_TCP_TA_DATA_STALL_CYCLES GRBM_GUI_ACTIVE",
    "tlb": "TCP_UTCL1_SERIALIZATION_STALL TCP_TOTAL_CACHE_ACCESSES TCP_UTCL1_STALL_INFLIGHT_MAX GRBM_GUI_ACTIVE",
}
STALL_COMMAND = ("rocprofv3 --pmc COUNTERS --output-format csv -d RUN_DIR/stall_WHO_PASS -o p -- python3 bench.py "
                 "KERNEL_ARGS --no-cpu-baseline --no-secondary --settle 0 --steps 5 --warmup 2")
WORKLOAD_FLAGS = ("--workload", "--secondary", "--no-secondary")


def workload_args(argv):
    """The workload flags (with their values) among bench.py's arguments."""
    out, it = [], iter(argv)
    for a in it:
        if a.split("=")[0] in WORKLOAD_FLAGS:
            out.append(a)
            if a in ("--workload", "--secondary"):
                out.append(next(it, ""))
    return " ".join(out)
KERNEL_SYMBOL = {"tile_": "gemm_tile_kernel", "skinny_": "gemm_skinny_kernel", "splitk_": "gemm_splitk_kernel",
                 # the split's first pass; its reduction is the short last kernel (for the hybrid: the
                 # data-parallel launch over the whole rounds)
                 "ksplit_tile_": "gemm_tile_kernel", "hybrid_": "gemm_tile_kernel", "streamk_": "gemm_tile_kernel",
                 # row bands: the large-tile launch over the whole rounds, then the rest on its own kernel
                 "band_": "gemm_tile_kernel",
                 "ksplit_": "gemm_skinny_kernel",
                 "masked_": "gemm_masked_kernel", "rowsum_wave": "rowsum_wave_kernel",
                 "rowsum_block": "rowsum_block_kernel"}


def _csv(path):
    import csv
    import glob

    files = glob.glob(path)
    if not files:
        raise SystemExit(f"--summarize: no file matches {path}")
    return list(csv.DictReader(open(files[0])))


def _counters(directory):
    """{kernel name: {counter: mean value per dispatch}} from one rocprofv3 --pmc run."""
    acc = {}
    for r in _csv(os.path.join(directory, "*counter_collection.csv")):
        d = acc.setdefault(r["Kernel_Name"], {})
        d.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in acc.items()}


def _pick(table, kernel):
    """The rocprofv3 kernel entry of a library kernel name (most frequent instantiation of its family)."""
    fam = next(v for k, v in KERNEL_SYMBOL.items() if kernel.startswith(k))
    names = [n for n in table if fam + "<" in n]
    if not names:
        raise SystemExit(f"--summarize: no {fam} entry")
    # equal counts (the hybrid's two launches): the data-parallel instance (last template argument 0)
    return max(names, key=lambda n: (table[n][1] if isinstance(table[n], tuple) else 0, ", 0>(" in n))


def summarize(run_dir):
    """Write profiles/ (kernel-trace and counter summaries, HBM traffic records) from one measurement run."""
    from workloads import lookup

    bench = json.load(open(os.path.join(run_dir, "bench.json")))
    jobs = [(bench["config"]["workload"], bench["roofline"]["kernel"], bench["ms_per_step"])]
    if "secondary" in bench:
        jobs.append((bench["secondary"]["workload"], bench["secondary"]["kernel"], bench["secondary"]["ms_per_step"]))
    src = bench.get("kernel_source_hash")
    per_kernel = bench.get("kernel_source_hashes", {})
    for _, kern, _ in jobs:
        if per_kernel.get(kern) != kernel_source_hash(kern):
            print(f"--summarize: the run measured {kern} from source {per_kernel.get(kern)}, the tree now holds "
                  f"{kernel_source_hash(kern)}; its traffic record will not be used by bench.py", file=sys.stderr)
    wargs = workload_args(bench.get("argv", []))
    cmd = lambda k: " ".join(("cd /tmp && " + PROFILE_COMMANDS[k].replace("WORKLOAD_ARGS", wargs)).split())  # noqa: E731
    stats = _csv(os.path.join(run_dir, "trace", "*kernel_stats.csv"))
    by_name = {r["Name"]: (r, int(r["Calls"])) for r in stats}
    out = os.path.join(ROOT, "profiles")
    os.makedirs(out, exist_ok=True)

    lines = ["# rocprofv3 --kernel-trace --stats summary (kernel_stats.csv), one MI355X",
             f"# command: {cmd('trace')}", f"# kernel source hash (bench.kernel_source_hash): {src}"]
    for wl, kern, _ in jobs:
        lines.append(f"# {wl}: {kern} = {_pick(by_name, kern)}")
    lines.append("# __amd_rocclr_copyBuffer = input uploads")
    # per-dispatch resources from the kernel trace: the run-time half of the zero-scratch check
    trace = _csv(os.path.join(run_dir, "trace", "*kernel_trace.csv"))
    res_cols = ("Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "LDS_Block_Size")
    resources = {}
    for r in trace:
        resources.setdefault(r["Kernel_Name"], set()).add(tuple(r.get(c, "?") for c in res_cols))
    for wl, kern, _ in jobs:
        sym = _pick(by_name, kern)
        for vals in sorted(resources.get(sym, ())):
            lines.append(f"# {kern} dispatch resources: " + ", ".join(f"{c} {v}" for c, v in zip(res_cols, vals)))
            if vals[0] not in ("0", "0.0"):
                raise SystemExit(f"--summarize: {kern} ran with Scratch_Size {vals[0]}")
    lines.append(",".join(f'"{c}"' for c in stats[0].keys()))
    for r in stats:
        lines.append(",".join(f'"{v}"' if k == "Name" else v for k, v in r.items()))
    name = "kernel_trace_stats__" + "__".join(j[0] for j in jobs) + ".txt"
    open(os.path.join(out, name), "w").write("\n".join(lines) + "\n")

    fetch, write = _counters(os.path.join(run_dir, "fetch")), _counters(os.path.join(run_dir, "write"))
    cal_f = _counters(os.path.join(run_dir, "cal_fetch"))
    cal_w = _counters(os.path.join(run_dir, "cal_write"))
    sq = _counters(os.path.join(run_dir, "sq"))
    copy_kib = 1024 * 1024  # --calibrate-copy 1024: 1 GiB read and written per copy
    copy_f = max(v["FETCH_SIZE"] for v in cal_f.values())
    copy_w = max(v["WRITE_SIZE"] for v in cal_w.values())
    fscale, wscale = copy_kib / copy_f, copy_kib / copy_w
    for wl, kern, ms in jobs:
        w = lookup(wl)
        trace_row = by_name[_pick(by_name, kern)][0]
        sym_f = _pick({n: (None, 1) for n in fetch}, kern)
        f_kib, w_kib = fetch[sym_f]["FETCH_SIZE"], write[_pick({n: (None, 1) for n in write}, kern)]["WRITE_SIZE"]
        c = sq[_pick({n: (None, 1) for n in sq}, kern)]
        hbm_r, hbm_w = f_kib * 1024 * fscale, w_kib * 1024 * wscale
        mops = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0) + c.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0)
        lds = c.get("SQ_LDS_IDX_ACTIVE", 0)
        txt = [f"# rocprofv3 counters for {kern} on {wl}, averages per dispatch, one MI355X",
               f"# kernel source hash: {per_kernel.get(kern)} ({kern}'s sources); {src} (all of csrc/)",
               f"# SQ counters: {cmd('sq')}",
               f"# FETCH_SIZE: {cmd('fetch')}",
               f"# WRITE_SIZE: {cmd('write')}",
               f"# copy calibration: {cmd('cal_fetch')} ; {cmd('cal_write')}",
               f"[{sym_f}]"]
        txt += [f"{k} = {v:.6g}" for k, v in sorted(c.items())]
        txt += [f"# LDS bank-conflict cycles / LDS active cycles = "
                f"{c.get('SQ_LDS_BANK_CONFLICT', 0) / lds if lds else 0:.3f}",
                (f"# MFMA ops x 512 = {mops * 512:.6g} (2*M*N*K*batch = {w.flops:.6g})" if mops else
                 "# no MFMA work"),
                f"FETCH_SIZE = {f_kib:.6g} KiB, WRITE_SIZE = {w_kib:.6g} KiB",
                f"# 1 GiB device copy: FETCH_SIZE = {copy_f:.6g} KiB, WRITE_SIZE = {copy_w:.6g} KiB "
                f"-> read scale {fscale:.3f}, write scale {wscale:.3f}",
                f"# HBM bytes per launch = {hbm_r + hbm_w:.6g} (read {hbm_r:.6g}, write {hbm_w:.6g}); "
                f"algorithmic {w.bytes:.6g} ({(hbm_r + hbm_w) / w.bytes:.2f}x)",
                f"# kernel-trace average {float(trace_row['AverageNs']) / 1e6:.4f} ms over {trace_row['Calls']} "
                f"calls; bench.py ms_per_step in the same run {ms:.4f} ms"]
        red = None
        if kern.endswith("+reduce"):
            # the split's second kernel: the workspace round trip (pass 1 writes the partials, pass 2 reads them)
            rname = lambda t: next((n for n in t if "tsm::" in n and "reduce_kernel<" in n), None)  # noqa: E731
            rf, rw, rt = rname(fetch), rname(write), rname(by_name)
            if rf and rw and rt:
                red = {"read": fetch[rf]["FETCH_SIZE"] * 1024 * fscale, "write": write[rw]["WRITE_SIZE"] * 1024 * wscale,
                       "avg_duration_ns": float(by_name[rt][0]["AverageNs"])}
                txt += [f"[{rf}]",
                        f"FETCH_SIZE = {fetch[rf]['FETCH_SIZE']:.6g} KiB, WRITE_SIZE = {write[rw]['WRITE_SIZE']:.6g} KiB",
                        f"# pass 2 HBM bytes = {red['read'] + red['write']:.6g} (read {red['read']:.6g}, write "
                        f"{red['write']:.6g}); kernel-trace average {red['avg_duration_ns'] / 1e6:.4f} ms",
                        f"# both passes: {hbm_r + hbm_w + red['read'] + red['write']:.6g} B per call "
                        f"({(hbm_r + hbm_w + red['read'] + red['write']) / w.bytes:.2f}x algorithmic)"]
        open(os.path.join(out, f"counters__{kern}__{wl}.txt"), "w").write("\n".join(txt) + "\n")
        rec = {"kernel": kern, "workload": wl, "source_hash": per_kernel.get(kern), "hbm_bytes_per_launch": hbm_r + hbm_w,
               "hbm_read_bytes_per_launch": hbm_r, "hbm_write_bytes_per_launch": hbm_w,
               "algorithmic_bytes_per_launch": w.bytes, "fetch_size_kib": f_kib, "write_size_kib": w_kib,
               "fetch_scale": fscale, "write_scale": wscale, "avg_duration_ns": float(trace_row["AverageNs"]),
               "calibration": f"FETCH_SIZE/WRITE_SIZE of a 1 GiB device-to-device copy (bench.py --calibrate-copy "
                              f"1024): {copy_f:.0f} KiB fetched, {copy_w:.0f} KiB written",
               "commands": [cmd("fetch"), cmd("write"), cmd("cal_fetch"), cmd("cal_write")]}
        if red:
            rec["pass2_hbm_bytes_per_call"] = red["read"] + red["write"]
            rec["pass2_avg_duration_ns"] = red["avg_duration_ns"]
        json.dump(rec, open(os.path.join(out, f"traffic_{wl}.json"), "w"), indent=1)
        print(f"{wl}: {kern}, HBM {hbm_r + hbm_w:.4g} B/launch ({(hbm_r + hbm_w) / w.bytes:.2f}x algorithmic)")
    if os.path.isdir(os.path.join(run_dir, "stall_ours_waits")):
        summarize_stalls(run_dir, jobs[0], src, per_kernel.get(jobs[0][1]))


def summarize_stalls(run_dir, job, src, kern_hash):
    """profiles/stall_counters__<kernel>__<workload>.txt: the STALL_PASSES counters of the headline kernel beside
    torch.matmul's, averaged over the dispatches after the first, with the ratios that locate lost MFMA cycles."""
    wl, kern, _ = job

    def load(who):
        vals = {}
        for ps in STALL_PASSES:
            rows = _csv(os.path.join(run_dir, f"stall_{who}_{ps}", "*counter_collection.csv"))
            fam = "Cijk" if who == "ref" else KERNEL_SYMBOL[next(k for k in KERNEL_SYMBOL if kern.startswith(k))] + "<"
            per = {}
            for r in rows:
                if fam in r["Kernel_Name"]:
                    per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            for c, xs in per.items():
                xs = xs[1:] if len(xs) > 1 else xs
                vals[(c, ps)] = sum(xs) / len(xs)
        return vals

    ours, ref = load("ours"), load("ref")
    cmd = lambda who, ps: " ".join(("cd /tmp && " + STALL_COMMAND.replace("COUNTERS", STALL_PASSES[ps])  # noqa: E731
                                    .replace("WHO", who).replace("PASS", ps)
                                    .replace("KERNEL_ARGS", "--torch-reference" if who == "ref" else "")).split())
    txt = [f"# where the MFMA pipes lose cycles: {kern} beside torch.matmul (hipBLASLt) on {wl}, one MI355X",
           f"# kernel source hash: {kern_hash} ({kern}'s sources); {src} (all of csrc/)",
           "# averages per dispatch over the dispatches after the first; one pass per counter group:"]
    txt += [f"#   {cmd('ours', ps)}" for ps in STALL_PASSES]
    txt += ["#   the same with --torch-reference for the torch.matmul column",
            f'"counter","pass","{kern}","torch.matmul"']
    for (c, ps) in sorted(ours):
        txt.append(f'"{c}","{ps}",{ours[(c, ps)]:.6g},{ref.get((c, ps), float("nan")):.6g}')

    def derived(v):
        g = v[("GRBM_GUI_ACTIVE", "waits")] / 8  # cycles per XCD
        wc = v[("SQ_WAVE_CYCLES", "waits")]
        return {"MFMA busy / (1024 SIMDs x cycles)": v[("SQ_VALU_MFMA_BUSY_CYCLES", "waits")] / (1024 * g),
                "SQ_WAIT_ANY / SQ_WAVE_CYCLES": v[("SQ_WAIT_ANY", "waits")] / wc,
                "L2 read latency (cycles)": v[("TCP_TCC_READ_REQ_LATENCY", "l1")] / v[("TCP_TCC_READ_REQ", "l1")],
                "VMEM latency (cycles)": v[("VmemLatency", "vmem_latency")],
                "LDS latency (cycles)": v[("LdsLatency", "lds_latency")]}
    do, dr = derived(ours), derived(ref)
    txt.append("# derived:")
    txt += [f"#   {k}: {do[k]:.3f} ({kern}) vs {dr[k]:.3f} (torch.matmul)" for k in do]
    name = f"stall_counters__{kern}__{wl}.txt"
    open(os.path.join(ROOT, "profiles", name), "w").write("\n".join(txt) + "\n")
    print(f"wrote profiles/{name}")


class Setup:
    """Inputs of one workload uploaded to the GPU, and a closure that runs one step."""

    def __init__(self, w, torch, tsm, act=0, slope=0.0, workspace=True):
        self.w = w
        self.act, self.slope = act, slope
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
        # a grouped workload carries per-problem row counts, uploaded once like the operands
        self.rows = w.rows() if hasattr(w, "rows") else None
        if self.rows is not None:
            self.rows_t = torch.from_numpy(self.rows).cuda()
            self.args = (w.M, w.N, w.K, self.a, self.lda, self.la, self.sA, self.b, self.ldb, self.lb, self.sB,
                         self.c, self.ldc, self.sC, self.rows_t, w.batch, self.code)
            self.kernel = tsm.tsm_gemm_grouped_kernel_name(*self.args)
            self.call = tsm.gemm_grouped
        else:
            self.args = (w.M, w.N, w.K, self.a, self.lda, self.la, self.sA, self.b, self.ldb, self.lb, self.sB,
                         self.c, self.ldc, self.sC, w.batch, self.code)
            self.kernel = tsm.tsm_gemm_kernel_name(*self.args)
            self.call = tsm.gemm_strided_batched_ex
            # few output tiles and deep K: split K through a workspace allocated here, outside the timed steps
            self.ws_bytes = tsm.gemm_workspace_bytes(w.M, w.N, w.K, w.batch) if workspace else 0
            if self.ws_bytes:
                self.ws = torch.empty(self.ws_bytes // 4, dtype=torch.float32, device="cuda")
                self.kernel = tsm.tsm_gemm_ws_kernel_name(*self.args, self.ws, self.ws_bytes)
                self.args = self.args + (act, slope, self.ws, self.ws_bytes)
                self.call = tsm.gemm_strided_batched_ws
            elif act:  # the same product with an activation fused into the epilogue
                self.args = self.args + (act, slope)
                self.call = tsm.gemm_strided_batched_act

    def step(self):
        self.call(*self.args, self.handle)

    def settle(self, seconds):
        """Run the step untimed for at least `seconds` of wall time (the GPU clock leaves its idle state)."""
        torch = self.torch
        t0, n = time.perf_counter(), 0
        while True:
            for _ in range(8):
                self.step()
            n += 8
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                return {"seconds": round(time.perf_counter() - t0, 3), "steps": n}

    def all_written(self):
        """One step over a NaN-filled C: every output element must come back finite (checked on the GPU)."""
        torch = self.torch
        self.c.fill_(float("nan"))
        self.step()
        torch.cuda.synchronize()
        if self.rows is not None:  # only the rows each group computes are written
            c = self.c.view(self.w.batch, self.w.M, self.w.N)
            ok = all(bool(torch.isfinite(c[g, :int(r)]).all()) for g, r in enumerate(self.rows))
        else:
            ok = bool(torch.isfinite(self.c).all())
        return ok

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
        if self.rows is not None:  # only the rows each group computes
            z = rng.choice(np.flatnonzero(self.rows > 0), ncells)
            i = (rng.random(ncells) * self.rows[z]).astype(np.int64)
        else:
            i = rng.integers(0, w.M, ncells)
        j = rng.integers(0, w.N, ncells)
        host = self.c.float().cpu().numpy().astype(np.float64).reshape(w.batch, w.M, w.N)
        got = host[z, i, j]
        ref, S = orc.gemm_points(self.A, self.B, w.M, w.N, w.K, w.in_fmt, z, i, j, strideA=self.A[0].size,
                                 strideB=self.B[0].size, a_layout=w.a_layout, b_layout=w.b_layout)
        ref = oracle.activate(ref, self.act, self.slope)
        bnd = oracle.bound(w.K, S, w.out_fmt, got, self.act, self.slope)
        ratio = float(np.max(np.abs(got - ref) / np.where(bnd > 0, bnd, 1.0)))
        return {"cells": ncells, "max_err_over_bound": ratio, "pass": bool(ratio <= 1.0 and np.all(np.isfinite(got)))}


def cpu_baseline(orc, w, A, B, target_s, max_s):
    """Oracle timed on problem 0 of the workload: the whole product when two short runs predict it takes at most
    max_s seconds, else whole output rows chosen for about target_s seconds.

    The short runs fit t(rows) = fixed + per_row * rows (the fixed part decodes B).
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
    full = fixed + per_row * w.M <= max_s
    rows = w.M if full else max(1, min(w.M, int((target_s - fixed) / per_row)))
    t = run(rows)
    flops = 2.0 * rows * w.N * w.K
    what = (f"the whole product of problem 0 ({w.M} x {w.N} x {w.K} fp64 multiply-adds" if full else
            f"rows 0..{rows - 1} of problem 0 ({rows} x {w.N} x {w.K} fp64 multiply-adds")
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": orc.threads(), "cpu": cpu_model(), "kind": "oracle",
            "sample": f"{what}, {t:.1f} s including the decode of B)", "seconds": t, "full_product": full}


def cpu_model() -> str:
    """The host CPU's model name, reported beside the oracle's thread count."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def rowsum_bench(args, w, torch, tsm):
    """Row-sum workload: one step is one rowsum call; HBM-bound, reported in GB/s."""
    import numpy as np

    import oracle

    log(f"generating {w.name} inputs on the host")
    X = w.operand()
    code = {"f32": tsm.TSM_ROWSUM_F32, "f16": tsm.TSM_ROWSUM_F16, "bf16": tsm.TSM_ROWSUM_BF16}[w.fmt]
    x = torch.from_numpy(X.view(np.float32 if w.fmt == "f32" else np.int16)).cuda()
    out = torch.empty(w.R, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    kernel = tsm.tsm_rowsum_kernel_name(w.R, w.C, x, w.C, 1, code, out)

    def time_steps(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            tsm.rowsum(w.R, w.C, x, w.C, 1, code, out, stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    time_steps(args.warmup)
    ms = time_steps(args.steps) / args.steps
    ms_i = statistics.median([(time_steps(12) - time_steps(2)) / 10 for _ in range(7)])
    orc = oracle.default()
    t0 = time.perf_counter()
    ref, S = orc.rowsum(X, w.R, w.C, w.C, 1, w.fmt)
    cpu_s = time.perf_counter() - t0
    got = out.cpu().numpy().astype(np.float64)
    ratio = float(np.max(np.abs(got - ref) / np.maximum(w.C * 2.0 ** -24 * S, 1e-300)))
    gbs = w.bytes / (ms * 1e-3) / 1e9
    return {
        "metric": "row-sum GB/s (% of MI355X HBM peak)", "value": gbs, "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.fmt, "data": "synthetic",
        "config": {"workload": w.name, "R": w.R, "C": w.C, "in": w.fmt, "seed": w.seed, "parallelism": "single GPU",
                   "accumulate": "f32"},
        "ms_per_step_interleaved_median": ms_i,
        "check": {"rows": w.R, "max_err_over_bound": ratio, "pass": bool(ratio <= 1.0 and np.all(np.isfinite(got)))},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": traffic_from_profiles(w.name, kernel), "kernel": kernel,
                     "algorithmic_bytes_per_launch": w.bytes, "algorithmic_flops_per_launch": w.flops},
        "cpu_baseline": {"value": w.bytes / cpu_s / 1e9, "unit": "GB/s", "cores": orc.threads(), "cpu": cpu_model(),
                         "kind": "oracle", "sample": f"all {w.R} rows, {cpu_s:.2f} s"},
        "kernel_source_hash": kernel_source_hash(), "kernel_source_hashes": {kernel: kernel_source_hash(kernel)},
        "argv": sys.argv[1:],
    }


def torch_reference(args, w, torch, tsm):
    """torch.matmul (hipBLASLt on ROCm) on the same seeded operands and layouts, timed like the benchmark's steps:
    a reference point for the library's number, never the reported value.  torch's product keeps the operand
    dtype (no float32 or cross-dtype output) and a batch runs as one batched product."""
    s = Setup(w, torch, tsm, workspace=False)
    dt = torch.bfloat16 if w.in_fmt == "bf16" else torch.float16

    def view(flat, layout, rows, cols, ld):
        # the logical rows x cols operand of each problem, as stored (row- or column-major)
        t = flat.view(dt).view(w.batch, -1)[:, :(cols if layout == "col" else rows) * ld]
        if layout == "col":
            return t.reshape(w.batch, cols, ld)[:, :, :rows].transpose(1, 2)
        return t.reshape(w.batch, rows, ld)[:, :, :cols]

    a = view(s.a, w.a_layout, w.M, w.K, s.lda)
    b = view(s.b, w.b_layout, w.K, w.N, s.ldb)
    if w.batch == 1:
        a, b = a[0], b[0]
    else:  # batched products in 16-bit with a transposed right operand: made contiguous first
        a, b = a.contiguous(), b.contiguous()
    s.step = lambda: torch.matmul(a, b)
    s.settle(args.settle)
    for _ in range(args.warmup):
        s.step()
    torch.cuda.synchronize()
    ms = s.time_steps(args.steps) / args.steps
    tflops = w.flops / (ms * 1e-3) / 1e12
    return {"reference": "torch.matmul", "torch": torch.__version__, "workload": w.name, "steps": args.steps,
            "ms_per_step": ms, "ms_per_step_interleaved_median": s.interleaved_ms(), "tflops": tflops,
            "pct_of_mfma_peak": 100.0 * tflops / MFMA_PEAK_TFLOPS, "out_dtype": str(dt).replace("torch.", "")}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="square_bf16_8192")
    ap.add_argument("--secondary", default="skinny_f16_16x16384x8192_b8")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of a sampled CPU baseline")
    ap.add_argument("--cpu-max-seconds", type=float, default=90.0,
                    help="time the oracle on the whole product when it is predicted to take at most this long")
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of untimed steps before the warm-up, so the GPU clock has left its idle state")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--torch-reference", action="store_true",
                    help="time torch.matmul on the workload's operands instead (a reference line, not the benchmark)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (to scale HBM counters)")
    ap.add_argument("--activation", choices=["none", "relu", "leaky_relu"], default="none",
                    help="fuse an activation into the epilogue (the result is checked through it)")
    ap.add_argument("--slope", type=float, default=0.01, help="leaky ReLU slope")
    ap.add_argument("--no-workspace", action="store_true",
                    help="never split K through a workspace (shapes with few output tiles then use split-K inside "
                         "a workgroup)")
    ap.add_argument("--summarize", metavar="RUN_DIR",
                    help="no GPU: write profiles/ from the rocprofv3 output of the commands in PROFILE_COMMANDS")
    args = ap.parse_args()

    if args.summarize:
        summarize(args.summarize)
        return

    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(sharding the product across GPUs by output slabs is not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch

    import tiled_shared_memory_amd as tsm
    from workloads import lookup

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
    w = lookup(args.workload)
    if hasattr(w, "operand"):  # a row-sum workload
        print(json.dumps(rowsum_bench(args, w, torch, tsm)), flush=True)
        return
    if args.torch_reference:
        print(json.dumps(torch_reference(args, w, torch, tsm)), flush=True)
        return
    act = {"none": 0, "relu": 1, "leaky_relu": 2}[args.activation]
    s = Setup(w, torch, tsm, act, args.slope if act == 2 else 0.0, workspace=not args.no_workspace)
    written = s.all_written()
    settle = s.settle(args.settle)
    log(f"kernel {s.kernel}; every output written: {written}; settled {settle['steps']} steps in "
        f"{settle['seconds']} s; warm-up {args.warmup}")
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
    check["every_output_written"] = written
    check["pass"] = bool(check["pass"] and written)
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
        "settle": settle,
        "check": check,
        "roofline": roof,
        "kernel_source_hash": kernel_source_hash(),
        "kernel_source_hashes": {s.kernel: kernel_source_hash(s.kernel)},
        "argv": sys.argv[1:],
    }
    if s.rows is not None:
        result["config"]["rows"] = s.rows.tolist()
    if act:
        result["config"]["activation"] = args.activation
        if act == 2:
            result["config"]["slope"] = args.slope
    # free the headline operands before the secondary workload
    s_main = s
    del s

    if not args.no_secondary and args.secondary:
        w2 = lookup(args.secondary)
        s2 = Setup(w2, torch, tsm)
        written2 = s2.all_written()
        s2.settle(args.settle)
        for _ in range(max(3, args.warmup // 2)):
            s2.step()
        torch.cuda.synchronize()
        n2 = max(10, args.steps // 2)
        ms2 = s2.time_steps(n2) / n2
        ms2i = s2.interleaved_ms()
        check2 = s2.check_cells(orc)
        check2["every_output_written"] = written2
        check2["pass"] = bool(check2["pass"] and written2)
        gbs2 = w2.bytes / (ms2 * 1e-3) / 1e9
        result["secondary"] = {
            "workload": w2.name, "kernel": s2.kernel, "ms_per_step": ms2, "ms_per_step_interleaved_median": ms2i,
            "hbm_gbs_algorithmic": gbs2, "pct_of_hbm_peak": 100.0 * gbs2 / HBM_PEAK_GBS,
            "tflops": w2.flops / (ms2 * 1e-3) / 1e12, "check": check2,
            "roofline": {"bound": "hbm", "achieved": gbs2, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs2 / HBM_PEAK_GBS, "traffic": traffic_from_profiles(w2.name, s2.kernel)},
        }
        result["kernel_source_hashes"][s2.kernel] = kernel_source_hash(s2.kernel)
        log(f"secondary {w2.name}: {ms2:.4f} ms, {gbs2:.0f} GB/s")
        del s2

    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(orc, w, s_main.A, s_main.B, args.cpu_seconds, args.cpu_max_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
