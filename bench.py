"""Benchmark: attention forward TFLOP/s and fraction of the MI355X bf16 dense MFMA peak.

Workload (one step = one fa_fwd call over the whole batch): causal attention forward, bf16,
B=8 H=32 N=4096 D=128, BHSD, Q/K/V ~ N(0,1) seeded (numpy default_rng([42, 3])), scale = 1/sqrt(128).
This is the batch-8, 4096-token inference shape of page ai6s.net/6a0d3bfb... (32 heads of 128).
FLOP per step = 4*B*H*N^2*D / 2 (causal) = 1.0995e12.

Prints ONE JSON line.  Besides the contract fields it carries:
  roofline      - the kernel's achieved TFLOP/s (algorithmic FLOP / mean launch time measured with
                  HIP events on the launch stream) against the bf16 dense peak 2516.6 TFLOP/s;
                  traffic = HBM bytes per launch from the committed rocprofv3 counter summary
                  (profiles/traffic_fa_fwd_c3.json) when it was taken on the current kernel source,
                  else null.
  cpu_baseline  - the fp64 oracle timed on a bounded sample of the same workload's rows on the host
                  cores, in the same unit; the sample also checks the timed GPU output (parity_sample).

Defaults: 50 untimed warm-up steps (the GPU clock settles over the first few tens of milliseconds),
then 100 timed steps.
Options: --gpus N (only 1 is supported), --steps K, --warmup W, --no-cpu-baseline,
         --calibrate-copy (after timing, run one plain device copy of 1 GiB for counter calibration).
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

METRIC = "attention fwd TFLOP/s + % of bf16 MFMA peak, causal B=8 H=32 N=4096 D=128"
PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fa_fwd_c3.json")
KERNEL_SOURCES = [os.path.join(ROOT, "transformer_attention_fwd_amd", "csrc", f)
                  for f in ("fa_kernels.hip", "fa_launch.h", "fa_api.cpp")]


def kernel_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--workload", default="c3", help=argparse.SUPPRESS)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this attention forward is measured on one GPU's share "
              "(--gpus %d, WORLD_SIZE=%d requested)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import transformer_attention_fwd_amd as fa
    from transformer_attention_fwd_amd import inputs

    w = inputs.WORKLOADS[args.workload]
    log("bench: generating %s inputs %s" % (w.name, (w.B, w.H, w.N, w.D)))
    qh, kh, vh = inputs.make_workload(w)
    dev = [torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda") for x in (qh, kh, vh)]
    q, k, v = dev
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    B, H, N, D = w.B, w.H, w.N, w.D
    layout = fa.LAYOUT_BHSD if w.layout == "BHSD" else fa.LAYOUT_BSND

    def step():
        st = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, D,
                       layout, w.causal, w.scale, fa.DTYPE_BF16, sptr)
        if st != fa.FA_OK:
            raise RuntimeError("fa_fwd failed: %s %s" % (fa.status_str(st), fa.last_error()))

    log("bench: warmup %d" % args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps, per-launch HIP events on the launch stream
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    launch_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    total_ms = evs[0].elapsed_time(evs[-1])
    ms_per_step = total_ms / args.steps
    flops = w.flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    mean_launch_ms = float(np.mean(launch_ms))
    achieved = flops / (mean_launch_ms * 1e-3) / 1e12
    log("bench: %d steps, %.4f ms/step (wall %.4f), median launch %.4f ms, best %.4f ms, %.1f TFLOP/s"
        % (args.steps, ms_per_step, (t1 - t0) * 1e3 / args.steps, float(np.median(launch_ms)), min(launch_ms), value))

    if args.calibrate_copy:
        n = 1 << 29  # 1 GiB of bf16
        src = torch.empty(n, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("bench: calibration copy of %d bytes done" % (2 * n))
        del src, dst

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        t = json.load(open(TRAFFIC_FILE))
        if t.get("kernel_sha") == kernel_sha() and t.get("workload") == w.name:
            traffic = t["hbm_bytes_per_launch"]
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "kernel": "fa_fwd_16<128,bf16,causal>", "mean_launch_ms": round(mean_launch_ms, 5),
                "kernel_sha": kernel_sha()}

    cpu_baseline = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle

        cores = min(16, os.cpu_count() or 1)
        torch.cuda.synchronize()
        # bounded sample: seeded rows, sized from a short calibration to about 12 s of wall time
        cal = inputs.sample_rows(B, H, N, 256, seed=900)
        t_a = time.perf_counter()
        oracle.attention_rows(qh, kh, vh, dtype="bf16", layout=w.layout, causal=w.causal, scale=w.scale,
                              rows=cal, nthreads=cores)
        t_cal = time.perf_counter() - t_a
        n_rows = int(min(B * H * N, max(512, 256 * 12.0 / max(t_cal, 1e-3))))
        rows = inputs.sample_rows(B, H, N, n_rows, seed=901)
        t_a = time.perf_counter()
        o_ref, lse_ref = oracle.attention_rows(qh, kh, vh, dtype="bf16", layout=w.layout, causal=w.causal,
                                               scale=w.scale, rows=rows, nthreads=cores)
        t_cpu = time.perf_counter() - t_a
        keys = (rows[:, 2] + 1) if w.causal else np.full(len(rows), N)
        sample_flops = float(np.sum(4.0 * D * keys))
        cpu_tflops = sample_flops / t_cpu / 1e12
        cpu_baseline = {"value": round(cpu_tflops, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                        "sample": "%d seeded query rows of the same workload (%.3e FLOP, %.1f s); full-step time "
                                  "at this rate %.0f s" % (len(rows), sample_flops, t_cpu, flops / (cpu_tflops * 1e12))}
        idx = torch.from_numpy(rows).to("cuda")
        o_s = o[idx[:, 0], idx[:, 1], idx[:, 2]].float().cpu().numpy().astype(np.float64)
        l_s = lse[idx[:, 0], idx[:, 1], idx[:, 2]].cpu().numpy().astype(np.float64)
        parity = {"rows": int(len(rows)), "max_abs_dO": float(np.abs(o_s - o_ref).max()),
                  "max_abs_dlse": float(np.abs(l_s - lse_ref).max())}
        log("bench: oracle %d rows in %.2f s on %d threads; parity max|dO| %.3e max|dlse| %.3e"
            % (len(rows), t_cpu, cores, parity["max_abs_dO"], parity["max_abs_dlse"]))

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal attention forward bf16 B=%d H=%d N=%d D=%d %s" % (B, H, N, D, w.layout),
                   "B": B, "H": H, "N": N, "D": D, "layout": w.layout, "causal": w.causal,
                   "scale": w.scale, "flop_per_step": flops},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline,
        "cpu_baseline": cpu_baseline,
        "parity_sample": parity,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
