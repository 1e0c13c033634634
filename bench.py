"""Benchmark of the semi-CRF hot path (one fwd+bwd = one step) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload nlp]

A step is one semicrf_fwd_bwd call (cumulative scores, the parallel-in-time
forward and backward sweeps over every checkpoint interval, data-parallel
posteriors, reductions) over one batch of seeded synthetic input already
resident in HBM.  The
default workload is the NLP-scale configuration (B=32, T=512, C=24, K=32).

Prints ONE JSON line on stdout:
  value      = B*T*K*C segment cells per second (whole job, 1 GPU)
  roofline   = the dominant kernel -- the parallel-in-time sweep (k_sweep_w
               for C <= 32, k_sweep otherwise; one launch per iteration) --
               as its algorithmic float64 FMA work divided by its time (HIP
               events the library records on the launch stream around the
               sweep phase during the timed steps), against the MI355X
               float64 vector peak (78.6 TFLOP/s); `traffic` is its HBM bytes
               per launch from rocprofv3 counters stored under profiles/ (null
               when absent or when the kernel sources changed since)
  cpu_baseline = the float64 oracle timed on this host on the same workload
  rates      = the fwd+bwd rate over valid positions (sum of L_b in place of
               B*T), and the semicrf_logz_fwd and semicrf_viterbi rates on the
               same input (timed after the fwd+bwd steps, same repetitions)
Diagnostics go to stderr.  --copy-calibration MB runs one device copy of MB
megabytes after the timed steps (outside them), the reference kernel for
scaling the FETCH_SIZE / WRITE_SIZE counters.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "semi-CRF fwd+bwd segment-cells/s (B*T*K*C) and % of roofline, 1 MI355X"
FP64_PEAK_TFLOPS = 78.6   # 256 CU x 64 lanes x 2 flop (FMA) x 2.4 GHz
HBM_PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "semi_markov_crf_zero_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def positions_and_kterms(lengths, K):
    """Sum over sequences of L_b and of sum_{t=1}^{L_b} min(K, t)."""
    npos = 0
    kterms = 0
    for L in lengths:
        L = int(L)
        npos += L
        if L >= K:
            kterms += K * (K + 1) // 2 + (L - K) * K
        else:
            kterms += L * (L + 1) // 2
    return npos, kterms


def algorithmic_flops(lengths, C, K):
    """Float64 flops the method itself needs per step (FMA = 2 flops):
    sweeps      forward and backward K-term sums (2 + 2 per segment cell) and
                the forward and backward C x C contractions (2 C^2 + 2 C^2 per
                position); the repeated parallel-in-time iterations and the
                verification are overhead of the design and not counted;
    posteriors  the duration posteriors (2 per segment cell) and the
                transition-posterior GEMM (2 C^2 per position)."""
    npos, kterms = positions_and_kterms(lengths, K)
    return {
        "sweeps": 4.0 * kterms * C + 4.0 * C * C * npos,
        "posteriors": 2.0 * kterms * C + 2.0 * C * C * npos,
    }


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


def cpu_baseline(inp, budget_s=12.0):
    import oracle

    oracle.core.build(force=False)
    cells = inp["B"] * inp["T"] * inp["K"] * inp["C"]
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count()
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.fwd_bwd(inp, nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el / reps * (reps + 1) > 3 * budget_s:
            break
    per = el / reps
    return {"value": cells / per, "unit": "segment-cells/s", "cores": threads, "kind": "oracle",
            "sample": "the full %s workload (B=%d T=%d C=%d K=%d), %d repetition(s) in %.1f s, "
                      "float64 C with OpenMP" % (inp["name"], inp["B"], inp["T"], inp["C"], inp["K"],
                                                 reps, el)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="nlp",
                    choices=["tiny", "nlp", "speech", "genome", "extreme"])
    ap.add_argument("--checkpoint-interval", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rates", action="store_true",
                    help="skip the logz / Viterbi timings (profiler runs of the fwd+bwd kernels)")
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="MB")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the batch would shard across GPUs with one all-reduce of the parameter "
              "gradients; see DESIGN.md). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from semi_markov_crf_zero_amd import binding as bd
    from semi_markov_crf_zero_amd.workloads import make_inputs

    inp = make_inputs(args.workload)
    inp["name"] = args.workload
    B, T, C, K = inp["B"], inp["T"], inp["C"], inp["K"]
    dev = torch.device("cuda:0")
    t = {k: torch.from_numpy(inp[k]).to(dev) for k in ("emissions", "lengths", "trans", "dur")}
    plan = bd.FwdBwdPlan(t["emissions"], t["lengths"], t["trans"], t["dur"],
                         checkpoint_interval=args.checkpoint_interval)
    ckpt = args.checkpoint_interval or bd.semicrf_checkpoint_interval(B, T, K)
    nph = len(bd.FWD_BWD_PHASES)
    for _ in range(args.warmup):
        plan.run()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nph + 1)]
              for _ in range(args.steps)]
    for evs in events:  # create the handles; the library re-records them
        for ev in evs:
            ev.record()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for i in range(args.steps):
        plan.run(phase_events=events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    phase_ms = np.zeros(nph)
    for evs in events:
        for p in range(nph):
            phase_ms[p] += evs[p].elapsed_time(evs[p + 1])
    phase_ms /= args.steps
    ms_step = wall * 1e3 / args.steps
    cells = float(B) * T * K * C
    value = cells / (ms_step * 1e-3)
    for name, ms in zip(bd.FWD_BWD_PHASES, phase_ms):
        log("phase %-18s %9.3f ms" % (name, ms))
    log("step %.3f ms (wall), %.3e segment-cells/s, workspace %.1f MB"
        % (ms_step, value, plan.ws_bytes / 1e6))

    # the other entry points on the same input, after (and outside) the
    # timed fwd+bwd steps: log Z alone and Viterbi, the same repetitions
    def timed(fn, reps):
        for _ in range(max(1, args.warmup)):
            fn()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t1) * 1e3 / reps

    valid = float(np.sum(np.asarray(inp["lengths"], dtype=np.int64))) * K * C
    rates = {"fwd_bwd_effective": valid / (ms_step * 1e-3),
             "unit": "segment-cells/s (effective: sum of L_b in place of B*T)"}
    if not args.no_rates:
        lz_ms = timed(bd.LogzPlan(t["emissions"], t["lengths"], t["trans"], t["dur"]).run,
                      args.steps)
        vt_ms = timed(bd.ViterbiPlan(t["emissions"], t["lengths"], t["trans"], t["dur"]).run,
                      args.steps)
        rates.update({"logz_fwd": cells / (lz_ms * 1e-3), "logz_fwd_ms": lz_ms,
                      "viterbi": cells / (vt_ms * 1e-3), "viterbi_ms": vt_ms})
        log("logz_fwd %.3f ms, viterbi %.3f ms" % (lz_ms, vt_ms))

    if args.copy_calibration > 0:
        n = int(args.copy_calibration * 1e6) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)  # an elementwise kernel: reads and writes 4n bytes
        torch.cuda.synchronize()
        log("copy calibration: %d bytes read, %d bytes written" % (4 * n, 4 * n))
        del src, dst

    flops = algorithmic_flops(inp["lengths"], C, K)
    # The dominant kernel is the sweep: one launch per parallel-in-time
    # iteration (at most one per checkpoint interval; those after convergence
    # return at once), so per launch the algorithmic work is the step's sweep
    # work over the launch count, and the average launch time is the phase
    # time over the same count -- the ratio is the phase rate.  The phase also
    # holds the small verification / fix-up kernels, so this is a lower bound.
    dom = "k_sweep_w" if C <= 32 else "k_sweep"
    nchunk = -(-T // ckpt)
    phase = float(phase_ms[1])
    achieved = flops["sweeps"] / (phase * 1e-3) / 1e12
    roofline = {"bound": "alu", "kernel": dom, "achieved": achieved, "peak": FP64_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / FP64_PEAK_TFLOPS,
                "traffic": stored_traffic(dom, args.workload),
                "launches_per_step": nchunk, "phase_ms": phase,
                "algorithmic_flops_per_step": flops["sweeps"]}
    out = {
        "metric": METRIC, "value": value, "unit": "segment-cells/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
        "data": "synthetic (seeded numpy PCG64, shapes of the pages' workloads)",
        "config": {"workload": args.workload, "B": B, "T": T, "C": C, "K": K,
                   "checkpoint_interval": ckpt, "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "phase_ms": {n: float(m) for n, m in zip(bd.FWD_BWD_PHASES, phase_ms)},
        "rates": rates,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
