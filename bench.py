"""Benchmark of the semi-CRF hot path (one fwd+bwd = one step) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload extreme]
                    [--sub speech,genome,nlp] [--no-cpu-baseline] [--no-peaks]

A step is one semicrf_fwd_bwd call (cumulative scores, the parallel-in-time
forward and backward sweeps over every checkpoint interval, data-parallel
posteriors, reductions) over one batch of seeded synthetic input already
resident in HBM.  The headline workload is the largest configuration,
extreme-scale (B=1, T=2^20, C=64, K=256); `sub` carries the same record for
the speech-, genome- and NLP-scale workloads (the ones the pages' speech /
genome claims are about), each timed the same way in the same run.

Prints ONE JSON line on stdout:
  value        B*T*K*C segment cells per second (whole job, 1 GPU)
  roofline     the dominant kernel -- the parallel-in-time sweep (k_sweep_w
               for C <= 32, k_sweep64 for C <= 64 and K <= 256, k_sweep256
               for C <= 256 and K <= 64, k_sweep otherwise) -- timed with
               HIP events the library records on the launch stream around
               its first launch
               (every checkpoint interval of both directions; once the
               verification passes, the later launches return at once and
               are timed with the rest of the phase).  Its algorithmic work
               in the units of the method's roofline: per segment cell and
               direction one transcendental (the log-sum-exp over durations)
               and 5 VALU operations, per position and direction a C x C
               contraction (2 C^2 flops).  `bound` names the resource with the
               longest roof time at the peaks below; `achieved` is that
               work over the measured time, `frac` = achieved / peak;
               `traffic` is the kernel's HBM bytes per launch from rocprofv3
               counters stored under profiles/ (null when absent or when the
               kernel sources changed since).
  scan_roofline  the score scan (the call's first phase) against the HBM peak:
               12 bytes per position and label (x read once, S written in
               float64) over the phase time.
  call_roofline  the same for the whole call (2 transcendentals and 12 VALU
               operations per cell, 6 C^2 flops per position, 20 bytes of
               HBM per position and label) against ms_per_step.
  peaks        measured on this GPU by libsemicrf_peaks.so (copy bandwidth,
               v_exp_f32, float64 / float32 FMA, float64 / bf16 MFMA) beside
               the published MI355X figures.
  memory       peak device memory of the headline run (torch's allocator:
               inputs, outputs, workspace -- the library allocates nothing)
               and the size the materialised edge tensor would have.
  cpu_baseline the float64 oracle timed on this host on a bounded sample of
               the headline workload (the first 2^17 positions for extreme).
  rates        fwd+bwd over valid positions, semicrf_logz_fwd and
               semicrf_viterbi on the same input (after the timed steps).
Diagnostics go to stderr.  --copy-calibration MB runs one device copy of MB
megabytes after the timed steps (outside them), the reference kernel for
scaling the FETCH_SIZE / WRITE_SIZE counters.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "semi-CRF fwd+bwd segment-cells/s (B*T*K*C) and % of roofline, 1 MI355X"
CSRC = os.path.join(ROOT, "semi_markov_crf_zero_amd", "csrc")
PEAKS_LIB = os.path.join(ROOT, "semi_markov_crf_zero_amd", "libsemicrf_peaks.so")

# Published MI355X figures (256 CUs at 2.4 GHz): the transcendental rate is
# a quarter of the float32 lane rate (16 per clock and CU).
VENDOR = {
    "hbm_GBs": 8000.0,
    "exp_T_per_s": 256 * 16 * 2.4e9 / 1e12,    # 9.83
    "valu_f32_Tops": 78.6,                      # 157.3 TFLOP/s = 78.6 T FMA (packed) per s
    "fp64_TFLOPs": 78.6,
    "fp32_TFLOPs": 157.3,
    "mfma_f32_TFLOPs": 157.3,
    "mfma_f64_TFLOPs": 78.6,
    "mfma_bf16_TFLOPs": 2500.0,
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def segment_cells(lengths, K, C):
    """Sum over sequences of sum_{t=1}^{L_b} min(K, t) * C (the segment
    cells of one direction) and the number of valid positions."""
    cells = 0
    npos = 0
    for L in lengths:
        L = int(L)
        npos += L
        kt = K * (K + 1) // 2 + (L - K) * K if L >= K else L * (L + 1) // 2
        cells += kt * C
    return cells, npos


def source_digest():
    """SHA-256 over every kernel source file (sorted by name)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()


def stored_traffic(kernel, workload):
    """HBM bytes per launch from profiles/traffic_<kernel>_<workload>.json, or
    None when absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != source_digest():
        return None
    return rec.get("bytes_per_launch")


# ---------------------------------------------------------------- peaks
def measure_peaks(dev):
    """Microbenchmarks of libsemicrf_peaks.so; {} when it is not built."""
    import torch

    if not os.path.exists(PEAKS_LIB):
        return {}
    lib = ctypes.CDLL(PEAKS_LIB)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.semicrf_peak_copy.argtypes = [P, P, Z, I, I, P, ctypes.POINTER(ctypes.c_float)]
    lib.semicrf_peak_alu.argtypes = [I, P, I, I, I, P, ctypes.POINTER(ctypes.c_float)]
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    ms = ctypes.c_float(0.0)
    out = {}
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    if lib.semicrf_peak_copy(src.data_ptr(), dst.data_ptr(), nbytes // 16, 8192, 5, st,
                             ctypes.byref(ms)) == 0:
        out["hbm_GBs"] = 2.0 * nbytes / (ms.value * 1e-3) / 1e9
    del src, dst
    grid, thr = 2048, 256
    buf = torch.empty(grid * thr, dtype=torch.float64, device=dev)
    # kind, iterations, operations per launch, scale to the reported unit
    specs = (
        ("exp_T_per_s", 0, 4096, grid * thr * 4096 * 8, 1e-12),
        ("fp64_TFLOPs", 1, 16384, grid * thr * 16384 * 8 * 2, 1e-12),
        ("fp32_TFLOPs", 2, 16384, grid * thr * 16384 * 8 * 2, 1e-12),
        ("mfma_f64_TFLOPs", 3, 2048, grid * 4 * 2048 * 4 * (2 * 16 * 16 * 4), 1e-12),
        ("mfma_bf16_TFLOPs", 4, 8192, grid * 4 * 8192 * 2 * (2 * 32 * 32 * 16), 1e-12),
    )
    for key, kind, iters, ops, scale in specs:
        if lib.semicrf_peak_alu(kind, buf.data_ptr(), grid, iters, 5, st, ctypes.byref(ms)) == 0:
            out[key] = ops / (ms.value * 1e-3) * scale
    torch.cuda.synchronize()
    return out


def pick(peaks, key):
    """Measured value when available (and positive), else the published one."""
    v = peaks.get(key)
    return (v, "measured") if v and v > 0 else (VENDOR[key], "published")


# ------------------------------------------------------------- roofline
def sweep_roofline(cells, npos, C, t_ms, peaks):
    """The sweep's algorithmic work (both directions) against the peaks."""
    exp_peak, exp_src = pick(peaks, "exp_T_per_s")
    valu_peak = VENDOR["valu_f32_Tops"]
    mfma_peak = VENDOR["mfma_f32_TFLOPs"]
    work = {"exp": 2.0 * cells, "valu": 10.0 * cells, "mfma": 4.0 * C * C * npos}
    roofs = {"exp": work["exp"] / (exp_peak * 1e12), "valu": work["valu"] / (valu_peak * 1e12),
             "mfma": work["mfma"] / (mfma_peak * 1e12)}
    gov = max(roofs, key=roofs.get)
    peak = {"exp": exp_peak, "valu": valu_peak, "mfma": mfma_peak}[gov]
    unit = {"exp": "Texp/s", "valu": "Tops/s", "mfma": "TFLOP/s"}[gov]
    achieved = work[gov] / (t_ms * 1e-3) / 1e12
    return {"bound": "alu" if gov != "mfma" else "mfma",
            "resource": {"exp": "transcendental unit (v_exp_f32)",
                         "valu": "float32 VALU", "mfma": "float32 MFMA"}[gov],
            "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
            "peak_source": exp_src if gov == "exp" else "published",
            "roof_ms": roofs[gov] * 1e3, "kernel_ms": t_ms,
            "work": {"transcendentals": work["exp"], "valu_ops": work["valu"],
                     "contraction_flops": work["mfma"]}}


def call_roofline(cells, npos, B, T, C, t_ms, peaks):
    exp_peak, _ = pick(peaks, "exp_T_per_s")
    hbm_peak, hbm_src = pick(peaks, "hbm_GBs")
    roofs = {"exp": 2.0 * cells / (exp_peak * 1e12),
             "valu": 12.0 * cells / (VENDOR["valu_f32_Tops"] * 1e12),
             "mfma": 6.0 * C * C * npos / (VENDOR["mfma_f32_TFLOPs"] * 1e12),
             "hbm": 20.0 * B * T * C / (hbm_peak * 1e9)}
    gov = max(roofs, key=roofs.get)
    return {"governing": gov, "roof_ms": roofs[gov] * 1e3, "ms": t_ms,
            "frac": roofs[gov] * 1e3 / t_ms, "roof_ms_by_resource": {k: v * 1e3 for k, v in roofs.items()}}


# --------------------------------------------------------- one workload
def run_workload(name, steps, warmup, ckpt, peaks, dev, want_rates, want_memory=False):
    import numpy as np
    import torch

    from semi_markov_crf_zero_amd import binding as bd
    from semi_markov_crf_zero_amd.workloads import make_inputs

    inp = make_inputs(name)
    B, T, C, K = inp["B"], inp["T"], inp["C"], inp["K"]
    if want_memory:
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats(dev)
        free0 = torch.cuda.mem_get_info(dev)[0]
        base_alloc = torch.cuda.memory_allocated(dev)
    t = {k: torch.from_numpy(inp[k]).to(dev) for k in ("emissions", "lengths", "trans", "dur")}
    plan = bd.FwdBwdPlan(t["emissions"], t["lengths"], t["trans"], t["dur"],
                         checkpoint_interval=ckpt)
    interval = ckpt or bd.semicrf_checkpoint_interval(B, T, C, K)
    nph = len(bd.FWD_BWD_PHASES)
    for _ in range(warmup):
        plan.run()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nph + 1)] for _ in range(steps)]
    for evs in events:  # create the handles; the library re-records them
        for ev in evs:
            ev.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        plan.run(phase_events=events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    phase_ms = np.zeros(nph)
    for evs in events:
        for p in range(nph):
            phase_ms[p] += evs[p].elapsed_time(evs[p + 1])
    phase_ms /= steps
    ms_step = wall * 1e3 / steps
    cells_bt = float(B) * T * K * C
    cells, npos = segment_cells(inp["lengths"], K, C)
    rec = {"workload": name, "B": B, "T": T, "C": C, "K": K, "checkpoint_interval": interval,
           "ms_per_step": ms_step, "segment_cells_per_s": cells_bt / (ms_step * 1e-3),
           "phase_ms": {n: float(m) for n, m in zip(bd.FWD_BWD_PHASES, phase_ms)}}
    # the sweep kernel the library runs at this shape
    dom = ("k_sweep_w" if C <= 32 else "k_sweep64" if C <= 64 and K <= 256
           else "k_sweep256" if C <= 256 and K <= 64 else "k_sweep")
    roof = sweep_roofline(cells, npos, C, float(phase_ms[1]), peaks)
    roof["kernel"] = dom
    roof["traffic"] = stored_traffic(dom, name)
    rec["roofline"] = roof
    rec["call_roofline"] = call_roofline(cells, npos, B, T, C, ms_step, peaks)
    # the score scan (phase 0) is HBM-bound: x read once (4 B) and S written in
    # float64 (8 B) per position and label, against the HBM peak
    hbm_peak, hbm_src = pick(peaks, "hbm_GBs")
    scan_gbs = 12.0 * B * T * C / (float(phase_ms[0]) * 1e-3) / 1e9
    rec["scan_roofline"] = {"bound": "hbm", "achieved": scan_gbs, "peak": hbm_peak, "unit": "GB/s",
                            "frac": scan_gbs / hbm_peak, "peak_source": hbm_src,
                            "bytes": 12.0 * B * T * C, "ms": float(phase_ms[0])}
    rec["effective_cells_per_s"] = float(np.sum(inp["lengths"], dtype=np.int64)) * K * C / (ms_step * 1e-3)
    log("%-8s step %8.3f ms  %.3e cells/s  sweep %.3f ms  roof frac %.3f (call %.3f)  phases %s"
        % (name, ms_step, rec["segment_cells_per_s"], phase_ms[1], roof["frac"],
           rec["call_roofline"]["frac"], " ".join("%.3f" % m for m in phase_ms)))
    if want_memory:
        torch.cuda.synchronize()
        rec["memory"] = {
            "peak_allocated_bytes": int(torch.cuda.max_memory_allocated(dev) - base_alloc),
            "device_free_delta_bytes": int(free0 - torch.cuda.mem_get_info(dev)[0]),
            "workspace_bytes": int(plan.ws_bytes),
            "inputs_bytes": int(sum(v.numel() * v.element_size() for v in t.values())),
            "edge_tensor_bytes_if_materialised": int(B) * T * K * C * C * 4,
        }
        log("memory: peak %.2f GB (workspace %.2f GB); the edge tensor would be %.1f TB"
            % (rec["memory"]["peak_allocated_bytes"] / 1e9, plan.ws_bytes / 1e9,
               rec["memory"]["edge_tensor_bytes_if_materialised"] / 1e12))
    if want_rates:
        def timed(fn, reps):
            for _ in range(max(1, warmup)):
                fn()
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            for _ in range(reps):
                fn()
            torch.cuda.synchronize()
            return (time.perf_counter() - t1) * 1e3 / reps

        lz_ms = timed(bd.LogzPlan(t["emissions"], t["lengths"], t["trans"], t["dur"]).run, steps)
        vt_ms = timed(bd.ViterbiPlan(t["emissions"], t["lengths"], t["trans"], t["dur"]).run,
                      steps)
        rec["rates"] = {"logz_fwd": cells_bt / (lz_ms * 1e-3), "logz_fwd_ms": lz_ms,
                        "viterbi": cells_bt / (vt_ms * 1e-3), "viterbi_ms": vt_ms}
        log("%-8s logz_fwd %.3f ms, viterbi %.3f ms" % (name, lz_ms, vt_ms))
    del plan, t
    torch.cuda.empty_cache()
    return rec, inp


def cpu_baseline(inp, name, max_positions=1 << 17, budget_s=12.0):
    import numpy as np

    import oracle

    oracle.core.build(force=False)
    T = min(inp["T"], max_positions)
    sample = dict(inp)
    if T < inp["T"]:
        sample["emissions"] = np.ascontiguousarray(inp["emissions"][:, :T])
        sample["lengths"] = np.minimum(inp["lengths"], T).astype(np.int32)
        sample["T"] = T
    cells = sample["B"] * T * sample["K"] * sample["C"]
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count()
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.fwd_bwd(sample, nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el / reps * (reps + 1) > 3 * budget_s:
            break
    per = el / reps
    what = ("the first %d positions of the %s workload" % (T, name) if T < inp["T"]
            else "the full %s workload" % name)
    return {"value": cells / per, "unit": "segment-cells/s", "cores": threads, "kind": "oracle",
            "sample": "%s (B=%d T=%d C=%d K=%d), %d repetition(s) in %.1f s, float64 C with "
                      "OpenMP" % (what, sample["B"], T, sample["C"], sample["K"], reps, el)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="extreme",
                    choices=["tiny", "nlp", "speech", "genome", "extreme"])
    ap.add_argument("--sub", default="speech,genome,nlp",
                    help="comma-separated workloads timed after the headline ('' for none)")
    ap.add_argument("--sub-steps", type=int, default=20)
    ap.add_argument("--checkpoint-interval", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true")
    ap.add_argument("--no-rates", action="store_true",
                    help="skip the logz / Viterbi timings (profiler runs of the fwd+bwd kernels)")
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="MB")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the "
              "batch, or for a single sequence its checkpoint intervals, would shard across "
              "GPUs with one all-reduce of the parameter gradients). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    dev = torch.device("cuda:0")
    peaks = {} if args.no_peaks else measure_peaks(dev)
    if peaks:
        log("peaks: " + ", ".join("%s %.1f" % kv for kv in peaks.items()))
    head, inp = run_workload(args.workload, args.steps, args.warmup, args.checkpoint_interval,
                             peaks, dev, not args.no_rates, want_memory=True)
    subs = {}
    for name in [s for s in args.sub.split(",") if s and s != args.workload]:
        subs[name], _ = run_workload(name, args.sub_steps, 3, 0, peaks, dev, not args.no_rates)

    if args.copy_calibration > 0:
        n = int(args.copy_calibration * 1e6) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)  # an elementwise kernel: reads and writes 4n bytes
        torch.cuda.synchronize()
        log("copy calibration: %d bytes read, %d bytes written" % (4 * n, 4 * n))
        del src, dst

    value = head["segment_cells_per_s"]
    out = {
        "metric": METRIC, "value": value, "unit": "segment-cells/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
        "data": "synthetic (seeded numpy PCG64, shapes of the pages' workloads)",
        "config": {"workload": args.workload, "B": head["B"], "T": head["T"], "C": head["C"],
                   "K": head["K"], "checkpoint_interval": head["checkpoint_interval"],
                   "parallelism": "none (1 GPU)"},
        "roofline": head["roofline"],
        "call_roofline": head["call_roofline"],
        "scan_roofline": head["scan_roofline"],
        "phase_ms": head["phase_ms"],
        "memory": head["memory"],
        "rates": dict(head.get("rates", {}), fwd_bwd_effective=head["effective_cells_per_s"]),
        "peaks": {"measured": peaks, "published": VENDOR},
        "sub": subs,
    }
    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(inp, args.workload)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
