"""Benchmark: attention forward TFLOP/s and fraction of the MI355X bf16 dense MFMA peak.

Workload (one step = one fa_fwd call over the whole batch): causal attention forward, bf16,
B=8 H=32 N=4096 D=128, BHSD, Q/K/V ~ N(0,1) seeded (numpy default_rng([42, 3])), scale = 1/sqrt(128).
This is the batch-8, 4096-token inference shape of page ai6s.net/6a0d3bfb... (32 heads of 128).
FLOP per step = 4*B*H*N^2*D / 2 (causal) = 1.0995e12.

Prints ONE JSON line.  Besides the contract fields it carries:
  roofline      - the attention kernel's achieved TFLOP/s (algorithmic FLOP / mean duration of its launches,
                  measured with HIP events on the launch stream) against the bf16 dense peak 2516.6 TFLOP/s;
                  traffic = HBM bytes per launch from the committed rocprofv3 counter summary
                  (profiles/traffic_fa_fwd_c3.json) when it was taken on the current kernel source, else null.
  cpu_baseline  - the fp64 oracle timed on a bounded sample of the same workload's rows on the host
                  cores (all the CPUs the process may use: the GPU machine's share of 16), in the same unit;
                  the sample also checks the timed GPU output (parity_sample).  The whole C3 oracle would
                  take about a minute at that rate; the sample keeps the default run within minutes.
  gpu_clock     - amd-smi's gfx clock (one value per XCD) and hotspot temperature before, during (sampled
                  in a thread while the timed steps run) and after; roofline.peak_at_measured_clock and
                  frac_at_measured_clock scale the peak by the mean clock seen during the run / 2400 MHz.
  config.flop_per_step is the metric's count (4*B*H*N^2*D, halved when causal) for whole problems, and
                  the visible (query, key) pairs x 4*D for windows, offsets and chunks;
                  config.flop_visible_pairs is the visible-pair count in every case (causal C3: N(N+1)/2
                  pairs per head, 0.024 % above N^2/2).

Defaults: 50 untimed warm-up steps (the GPU clock settles over the first few tens of milliseconds),
then about 3 s of timed steps (the count from the warm-up's pace; --steps overrides).
Options: --gpus N (only 1 is supported), --steps K, --warmup W, --no-cpu-baseline,
         --calibrate-copy (after timing, run one plain device copy of 1 GiB for counter calibration),
         --workload NAME: c3 (default), or one of the variants of the same C3 tensors:
           c3_split4      the keys in 4 chunks of 1024 (fa_fwd_ex per chunk) combined by fa_merge
           c3_window1024  causal with a sliding window of 1024 earlier keys
           prefill_cache  the last 1024 queries against all 4096 keys (bottom-right causal, q_offset 3072)
           c3_noncausal   the same tensors without the causal mask (the ping-pong kernel; with c3 it gives
                          the causal speed-up the catlass page tabulates in "Causal Mask的实现差异")
         or c4 / c5 (the plain causal forward on those configurations), or c1 (fp32, non-causal, B=1 H=2
           N=512 D=64 BSND: its rate against the 157.3 TFLOP/s fp32 MFMA peak),
         or varlen: one step = one fa_fwd_varlen over 8 packed causal sequences (H=32 D=128 bf16) whose
           lengths are drawn uniformly from [512, 7680] (mean 4096: the C3 batch as a length mix),
         or c3_bwd: one step = one fa_bwd (dQ, dK, dV) on the C3 tensors with a seeded upstream gradient
           (O and lse from one fa_fwd before timing).  FLOP per step = the five products of the backward
           (recomputed S, dP, dV, dK, dQ) over the visible pairs, 10*D per pair = 2.5 x the forward's,
         or c3_bwd_window1024: the same through fa_bwd_ex with a sliding window of 1024 earlier keys
           (O and lse from fa_fwd_ex with that window),
         or c3_bwd_fp32: fa_bwd on the C3 draws kept in fp32 (roofline against the fp32 MFMA peak),
         or c3_bwd_atomic: fa_bwd_atomic on the c3_bwd tensors (dQ summed with fp32 atomic adds inside the
           dK/dV kernel instead of a second pass over the keys),
         or varlen_bwd: one step = one fa_bwd_varlen on the varlen workload's packed sequences with a
           seeded upstream gradient (O and lse from one fa_fwd_varlen before timing).
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
PEAK_HBM_GBS = 8000.0
PEAK_FP32_TFLOPS = 157.3  # dense fp32 MFMA
MAX_GFX_MHZ = 2400.0  # the clock the peaks are quoted at
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fa_fwd_c3.json")
KERNEL_SOURCES = [os.path.join(ROOT, "transformer_attention_fwd_amd", "csrc", f)
                  for f in ("fa_kernels.hip", "fa_device.h", "fa_launch.h")]
VARIANTS = {
    "c3": dict(desc="causal", window=-1, chunks=1, nq=None),
    "c3_split4": dict(desc="causal, keys in 4 chunks + lse merge", window=-1, chunks=4, nq=None),
    "c3_window1024": dict(desc="causal, sliding window 1024", window=1024, chunks=1, nq=None),
    "prefill_cache": dict(desc="causal, last 1024 queries vs 4096 cached keys", window=-1, chunks=1, nq=1024),
    "c3_noncausal": dict(desc="non-causal", window=-1, chunks=1, nq=None, causal=False),
}


def kernel_sha() -> str:
    """Hash of the forward kernel's source with // comments and blank lines removed (code changes only)."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        for line in open(p, encoding="utf-8").read().splitlines():
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def fwd_kernel_label(nq, nk, q_offset, window, chunks, causal=True, dtype="bf16", d=128):
    """Which forward kernel a call runs, by the library's own rule: fp32 runs fa_fwd_32; a 16-bit non-causal call
    whose query and key counts are multiples of 256 runs the ping-pong kernel; a whole causal problem pairs
    256-query tiles (8 waves) when ceil(N/256) and ceil(N/64) are even, on the ping-pong kernel when N is also
    a multiple of 256, else 128-query tiles (4 waves) when ceil(N/128) and ceil(N/64) are even; a key chunk
    that starts at a query row runs on the ping-pong kernel split into row ranges (chunk_splits); every other
    call runs one 128-query tile per workgroup."""
    if dtype == "fp32":
        return "fa_fwd_32<%d,%s>" % (d, "causal" if causal else "non-causal")
    if not causal:
        if nq % 256 == 0 and nk % 256 == 0:
            return "fa_fwd_16pp<%d,bf16,non-causal> (ping-pong, 8 waves)" % d
        return "fa_fwd_16<%d,bf16,non-causal> (one 128-query tile per workgroup, 4 waves)" % d
    if window >= 0:
        return "fa_fwd_16<%d,bf16,causal,window> (4 waves)" % d
    if chunks > 1:
        if all(chunk_splits(nq, nk, q_offset, chunks)):
            return ("fa_fwd_16pp<%d,bf16,causal,pair,chunk> per key chunk (ping-pong, 8 waves: the chunk's square "
                    "as heavy/light pairs, the rows after it in chains of full units, O = 0 for the rows before it)"
                    % d)
        return "fa_fwd_16<%d,bf16,causal> (one 128-query tile per workgroup, 4 waves) per key chunk" % d
    if chunks == 1 and q_offset == 0 and nq == nk and (nq + 63) // 64 % 2 == 0:
        if (nq + 255) // 256 % 2 == 0:
            if nq % 256 == 0:
                return "fa_fwd_16pp<%d,bf16,causal> (ping-pong, paired 256-query tiles, 8 waves)" % d
            return "fa_fwd_16<%d,bf16,causal> (paired 256-query tiles, 8 waves)" % d
        if (nq + 127) // 128 % 2 == 0:
            return "fa_fwd_16<%d,bf16,causal> (paired 128-query tiles, 4 waves)" % d
    return "fa_fwd_16<%d,bf16,causal> (one 128-query tile per workgroup, 4 waves)" % d


def chunk_splits(nq, nk, q_offset, chunks):
    """Per key chunk of a causal call: whether the library's rule runs it on the ping-pong kernel split into
    row ranges (rows before the chunk's first key, its square, the rows after it) rather than on fa_fwd_16:
    the chunk length a multiple of 512, its first key at a query row (q_offset <= kv_start) and the rows
    after the square a multiple of 256.  Either way a chunk is one launch."""
    out = []
    for c in range(chunks):
        a, b = nk * c // chunks, nk * (c + 1) // chunks
        i0, kv_len = a - q_offset, b - a
        rest = nq - i0 - kv_len
        out.append(i0 >= 0 and kv_len > 0 and kv_len % 512 == 0 and rest >= 0 and rest % 256 == 0)
    return out


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def visible_keys(nq, nk, q_offset, window):
    """Keys each query row sees (causal, optional window): array of length nq."""
    import numpy as np
    qpos = q_offset + np.arange(nq, dtype=np.int64)
    hi = np.minimum(qpos, nk - 1)
    lo = np.maximum(0, qpos - window) if window >= 0 else np.zeros(nq, dtype=np.int64)
    return np.maximum(hi - lo + 1, 0)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def smi_sample():
    """GPU 0's gfx clocks (MHz, one per XCD) and hotspot temperature from amd-smi, or an error string.

    Under rocprofv3 (ROCPROFILER_LIBRARY_CTOR set) nothing is sampled: the profiler's preloaded library
    would start up inside the amd-smi child, which then starts its interpreter from a process that has
    already touched the GPU."""
    import subprocess
    if os.environ.get("ROCPROFILER_LIBRARY_CTOR"):
        return {"t": round(time.time(), 2), "error": "not sampled under a profiler"}
    try:
        out = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "-t", "--json"], stdout=subprocess.PIPE,
                             stderr=subprocess.PIPE, text=True, timeout=30)
        d = json.loads(out.stdout)["gpu_data"][0]
        clocks = [v["clk"]["value"] for k, v in sorted(d["clock"].items()) if k.startswith("gfx_")]
        temp = d["temperature"].get("hotspot", {})
        return {"t": round(time.time(), 2), "gfx_mhz": clocks, "hotspot_c": temp.get("value") if isinstance(temp, dict)
                else None}
    except Exception as e:  # no amd-smi, no permission, another format: say so instead of guessing
        return {"t": round(time.time(), 2), "error": "%s: %s" % (type(e).__name__, str(e)[:120])}


class ClockSampler:
    """amd-smi samples before, during (a background thread, one sample after another) and after a timed loop."""

    def __enter__(self):
        import threading
        self.before = smi_sample()
        self.during = []
        self._stop = threading.Event()

        def loop():
            while not self._stop.is_set():
                self.during.append(smi_sample())
                self._stop.wait(0.2)
        self._thread = threading.Thread(target=loop, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join(timeout=60)
        self.after = smi_sample()
        return False

    def mean_clock_during(self):
        """Mean gfx clock over the samples taken while the steps ran.  amd-smi refreshes its reading about once a
        second, so the first samples can still repeat the idle reading taken before the run: those are left out."""
        stale = self.before.get("gfx_mhz")
        vals = [sum(x["gfx_mhz"]) / len(x["gfx_mhz"]) for x in self.during if x.get("gfx_mhz") and x["gfx_mhz"] != stale]
        return sum(vals) / len(vals) if vals else None

    def report(self):
        return {"before": self.before, "during": self.during, "after": self.after,
                "mean_gfx_mhz_during": self.mean_clock_during(), "max_gfx_mhz": MAX_GFX_MHZ}


def finish_line(line, clocks):
    """Clock samples, the fraction of the peak at the measured clock, and the host (for every bench line)."""
    line["gpu_clock"] = clocks.report()
    mhz = clocks.mean_clock_during()
    roof = line.get("roofline") or {}
    if mhz and roof.get("peak"):
        adj = roof["peak"] * mhz / MAX_GFX_MHZ
        roof["peak_at_measured_clock"] = round(adj, 1)
        roof["frac_at_measured_clock"] = round(roof["achieved"] / adj, 4)
    line["host"] = {"cpu_model": cpu_model(), "cpus": os.cpu_count()}


def choose_steps(args, step_ms):
    """--steps if given, else enough steps for about 3 s of timed work (20 to 5000)."""
    if args.steps:
        return args.steps
    return int(min(5000, max(20, round(3000.0 / max(step_ms, 1e-3)))))


def warmup_ms(step, n, torch):
    """Run n warm-up steps; return the mean ms of the last half of them (wall clock, synchronised)."""
    for _ in range(max(1, n // 2)):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    k = max(1, n - n // 2)
    for _ in range(k):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / k


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0, help="timed steps (default: about 3 s of work)")
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--workload", default="c3")
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

    if args.workload in ("c3_bwd", "c3_bwd_window1024", "c3_bwd_fp32", "c3_bwd_atomic"):
        return bench_bwd(args, window=1024 if args.workload == "c3_bwd_window1024" else -1,
                         dtype="fp32" if args.workload == "c3_bwd_fp32" else "bf16",
                         atomic=args.workload == "c3_bwd_atomic")
    if args.workload == "varlen":
        return bench_varlen(args)
    if args.workload == "varlen_bwd":
        return bench_varlen_bwd(args)
    if args.workload in VARIANTS:
        var = VARIANTS[args.workload]
        w = inputs.WORKLOADS["c3"]
    elif args.workload in ("c1", "c4", "c5"):
        var = VARIANTS["c3"]
        w = inputs.WORKLOADS[args.workload]
    else:
        raise SystemExit("unknown workload %s" % args.workload)
    if var.get("causal") is False:
        import dataclasses
        w = dataclasses.replace(w, causal=False)
    dtype = w.dtypes[0]  # bf16, or fp32 for c1
    dcode = fa.DTYPE_FP32 if dtype == "fp32" else fa.DTYPE_BF16
    peak = PEAK_FP32_TFLOPS if dtype == "fp32" else PEAK_BF16_TFLOPS
    log("bench: generating %s inputs %s" % (w.name, (w.B, w.H, w.N, w.D)))
    qh, kh, vh = inputs.make_workload(w)
    B, H, N, D = w.B, w.H, w.N, w.D
    Nk = N
    Nq = var["nq"] or N
    q_offset = Nk - Nq
    if Nq != N:
        qh = np.ascontiguousarray(qh[:, :, N - Nq:, :])  # BHSD: the last Nq query rows
    window, chunks = var["window"], var["chunks"]
    if dtype == "fp32":
        to_dev = lambda x: torch.from_numpy(x).to("cuda")
    else:
        to_dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda")
    q, k, v = to_dev(qh), to_dev(kh), to_dev(vh)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    layout = fa.LAYOUT_BHSD if w.layout == "BHSD" else fa.LAYOUT_BSND
    bounds = [Nk * c // chunks for c in range(chunks + 1)]
    if chunks > 1:
        o_parts = torch.empty((chunks,) + tuple(q.shape), dtype=q.dtype, device="cuda")
        l_parts = torch.empty((chunks, B, H, Nq), dtype=torch.float32, device="cuda")

    def check(st, what):
        if st != fa.FA_OK:
            raise RuntimeError("%s failed: %s %s" % (what, fa.status_str(st), fa.last_error()))

    def attention_launches():
        if chunks == 1 and window < 0 and Nq == Nk:
            check(fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, D,
                            layout, w.causal, w.scale, dcode, sptr), "fa_fwd")
        elif chunks == 1:
            check(fa.fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Nq, Nk,
                               D, layout, w.causal, window, q_offset, 0, Nk, w.scale, dcode, sptr), "fa_fwd_ex")
        else:
            for c in range(chunks):
                check(fa.fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_parts[c].data_ptr(),
                                   l_parts[c].data_ptr(), B, H, Nq, Nk, D, layout, w.causal, window, q_offset,
                                   bounds[c], bounds[c + 1] - bounds[c], w.scale, dcode, sptr), "fa_fwd_ex")

    def merge_launch():
        check(fa.fa_merge(o_parts.data_ptr(), l_parts.data_ptr(), chunks, o.data_ptr(), lse.data_ptr(), B, H, Nq, D,
                          layout, dcode, sptr), "fa_merge")

    def whole_step():
        attention_launches()
        if chunks > 1:
            merge_launch()

    log("bench: warmup %d" % args.warmup)
    args.steps = choose_steps(args, warmup_ms(whole_step, args.warmup, torch))

    # timed region: K steps; HIP events on the launch stream around the attention launches and the merge
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    with ClockSampler() as clocks:
        t0 = time.perf_counter()
        for i in range(args.steps):
            ev[i][0].record(stream)
            attention_launches()
            ev[i][1].record(stream)
            if chunks > 1:
                merge_launch()
            ev[i][2].record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    attn_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(args.steps)]
    merge_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in range(args.steps)]
    total_ms = ev[0][0].elapsed_time(ev[-1][2])
    ms_per_step = total_ms / args.steps
    # whole problems: the metric's own count, 4*B*H*N^2*D halved when causal; otherwise the visible pairs
    pairs_flops = float(4.0 * D * B * H * visible_keys(Nq, Nk, q_offset, window).sum()) if w.causal else w.flops()
    whole = chunks == 1 and window < 0 and Nq == Nk
    flops = w.flops() if whole else pairs_flops
    value = flops / (ms_per_step * 1e-3) / 1e12
    mean_attn_ms = float(np.mean(attn_ms))
    achieved = flops / (mean_attn_ms * 1e-3) / 1e12
    log("bench: %d steps, %.4f ms/step (wall %.4f), attention median %.4f ms best %.4f ms, %.1f TFLOP/s"
        % (args.steps, ms_per_step, (t1 - t0) * 1e3 / args.steps, float(np.median(attn_ms)), min(attn_ms), value))

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
    if os.path.exists(TRAFFIC_FILE) and args.workload == "c3":
        t = json.load(open(TRAFFIC_FILE))
        if t.get("kernel_sha") == kernel_sha() and t.get("workload") == w.name:
            traffic = t["hbm_bytes_per_launch"]
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic,
                "kernel": fwd_kernel_label(Nq, Nk, q_offset, window, chunks, w.causal, dtype, D),
                "mean_launch_ms": round(mean_attn_ms / chunks, 5),
                "launches_per_step": chunks,
                "kernel_sha": kernel_sha()}
    extra = {}
    if chunks > 1:
        # the merge reads every part's O and lse once and writes O and lse once
        mbytes = (chunks + 1) * (B * H * Nq * D * 2 + B * H * Nq * 4)
        mean_merge_ms = float(np.mean(merge_ms))
        gbs = mbytes / (mean_merge_ms * 1e-3) / 1e9
        extra["merge_roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                   "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                                   "kernel": "fa_merge_kernel<bf16,128>", "mean_launch_ms": round(mean_merge_ms, 5),
                                   "bytes_per_launch": mbytes}

    cpu_baseline = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle

        cores = len(os.sched_getaffinity(0))  # the CPUs this process may use (the GPU machine: 16)
        torch.cuda.synchronize()
        ref = lambda rows: oracle.attention_rows_ex(qh, kh, vh, dtype=dtype, layout=w.layout, causal=w.causal,
                                                    scale=w.scale, rows=rows, window=window, q_offset=q_offset,
                                                    nthreads=cores)
        # bounded sample: seeded rows, sized from a short calibration (after one warm call, which pays the
        # library load and thread start-up) to about 15 s of wall time
        cal = inputs.sample_rows(B, H, Nq, 1024, seed=900)
        ref(cal[:64])
        t_a = time.perf_counter()
        ref(cal)
        t_cal = time.perf_counter() - t_a
        n_rows = int(min(B * H * Nq, max(512, len(cal) * 15.0 / max(t_cal, 1e-3))))
        rows = inputs.sample_rows(B, H, Nq, n_rows, seed=901)
        t_a = time.perf_counter()
        o_ref, lse_ref = ref(rows)
        t_cpu = time.perf_counter() - t_a
        keys = visible_keys(Nq, Nk, q_offset, window)[rows[:, 2]] if w.causal else np.full(len(rows), Nk)
        sample_flops = float(np.sum(4.0 * D * keys))
        cpu_tflops = sample_flops / t_cpu / 1e12
        cpu_baseline = {"value": round(cpu_tflops, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                        "cpu_model": cpu_model(),
                        "sample": "%d seeded query rows of the same workload (%.3e FLOP, %.1f s); full-step time "
                                  "at this rate %.0f s" % (len(rows), sample_flops, t_cpu, flops / (cpu_tflops * 1e12))}
        idx = torch.from_numpy(rows).to("cuda")  # (b, h, i) triples; O is [B][H][N][D] or [B][N][H][D]
        if w.layout == "BHSD":
            o_s = o[idx[:, 0], idx[:, 1], idx[:, 2]].float().cpu().numpy().astype(np.float64)
        else:
            o_s = o[idx[:, 0], idx[:, 2], idx[:, 1]].float().cpu().numpy().astype(np.float64)
        l_s = lse[idx[:, 0], idx[:, 1], idx[:, 2]].cpu().numpy().astype(np.float64)
        err = np.abs(o_s - o_ref)
        # the bf16 bound: |dO| <= max(1e-2, one bf16 ulp of the exact value) per element (an output rounded
        # to bf16 can sit half an ulp away before any other error)
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(o_ref), 2.0 ** -126))) - 7)
        parity = {"rows": int(len(rows)), "max_abs_dO": float(err.max()),
                  "max_abs_dlse": float(np.abs(l_s - lse_ref).max()),
                  "elements_over_1e-2": int(np.sum(err > 1e-2)),
                  "elements_over_max_1e-2_ulp": int(np.sum(err > np.maximum(1e-2, ulp)))}
        log("bench: oracle %d rows in %.2f s on %d threads; parity max|dO| %.3e max|dlse| %.3e"
            % (len(rows), t_cpu, cores, parity["max_abs_dO"], parity["max_abs_dlse"]))

    if args.workload == "c3":
        metric = METRIC
        workload = "causal attention forward bf16 B=%d H=%d N=%d D=%d %s" % (B, H, N, D, w.layout)
    elif args.workload in ("c1", "c4", "c5"):
        metric = "attention fwd TFLOP/s, %s %s, B=%d H=%d N=%d D=%d" % ("causal" if w.causal else "non-causal", dtype,
                                                                      B, H, N, D)
        workload = "%s attention forward %s B=%d H=%d N=%d D=%d %s" % ("causal" if w.causal else "non-causal", dtype,
                                                                      B, H, N, D, w.layout)
    else:
        metric = "attention fwd TFLOP/s, %s, B=%d H=%d Nq=%d Nk=%d D=%d" % (var["desc"], B, H, Nq, Nk, D)
        workload = "attention forward bf16 %s B=%d H=%d Nq=%d Nk=%d D=%d %s" % (var["desc"], B, H, Nq, Nk, D,
                                                                              w.layout)
    config = {"workload": workload, "B": B, "H": H, "N": N, "D": D, "layout": w.layout, "causal": w.causal,
              "scale": w.scale, "flop_per_step": flops, "flop_visible_pairs": pairs_flops}
    if args.workload != "c3":
        config.update({"Nq": Nq, "Nk": Nk, "q_offset": q_offset, "window": window, "kv_chunks": chunks})
    line = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": config,
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "pct_of_dtype_peak": round(100.0 * value / peak, 2),
        "roofline": roofline,
        "cpu_baseline": cpu_baseline,
        "parity_sample": parity,
    }
    line.update(extra)
    finish_line(line, clocks)
    print(json.dumps(line), flush=True)


def bench_varlen(args):
    """One step = fa_fwd_varlen over a seeded causal length mix; see the module notes."""
    import numpy as np
    import torch

    import transformer_attention_fwd_amd as fa
    from transformer_attention_fwd_amd import inputs

    B, H, D = 8, 32, 128
    lens = inputs.varlen_lengths(B, 512, 7680, seed=3)
    cu = inputs.cu_seqlens(lens)
    total = int(cu[-1])
    scale = float(np.float32(1.0 / np.sqrt(D)))
    log("bench: varlen lengths %s (total %d)" % (list(lens), total))
    qh, kh, vh = inputs.make_varlen(lens, lens, H, D, dtype="bf16", seed=3)
    to_dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda")
    q, k, v = to_dev(qh), to_dev(kh), to_dev(vh)
    cu_d = torch.from_numpy(cu).to("cuda")
    o = torch.empty_like(q)
    lse = torch.empty((H, total), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    max_q = int(lens.max())

    def step():
        st = fa.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), cu_d.data_ptr(),
                              cu_d.data_ptr(), B, H, total, total, max_q, D, True, scale, fa.DTYPE_BF16,
                              stream.cuda_stream)
        if st != fa.FA_OK:
            raise RuntimeError("fa_fwd_varlen failed: %s %s" % (fa.status_str(st), fa.last_error()))

    log("bench: warmup %d" % args.warmup)
    args.steps = choose_steps(args, warmup_ms(step, args.warmup, torch))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    with ClockSampler() as clocks:
        t0 = time.perf_counter()
        for i in range(args.steps):
            ev[i][0].record(stream)
            step()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    call_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(args.steps)]
    ms_per_step = ev[0][0].elapsed_time(ev[-1][1]) / args.steps
    pairs = float(H * sum(int(n) * (int(n) + 1) // 2 for n in lens))
    flops = 4.0 * D * pairs
    value = flops / (ms_per_step * 1e-3) / 1e12
    mean_ms = float(np.mean(call_ms))
    achieved = flops / (mean_ms * 1e-3) / 1e12
    log("bench: %d steps, %.4f ms/step (wall %.4f), median %.4f ms, %.1f TFLOP/s"
        % (args.steps, ms_per_step, (t1 - t0) * 1e3 / args.steps, float(np.median(call_ms)), value))
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "kernel": "fa_fwd_16<128,bf16,causal,varlen>", "mean_launch_ms": round(mean_ms, 5),
                "launches_per_step": 1}
    cpu_baseline = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle

        cores = len(os.sched_getaffinity(0))  # the CPUs this process may use (the GPU machine: 16)
        rng = np.random.default_rng([4242, 3, 12])
        t_cpu, n_rows, sample_flops = 0.0, 0, 0.0
        err_o, err_l = 0.0, 0.0
        o_h = o.float().cpu().numpy().astype(np.float64)
        l_h = lse.cpu().numpy().astype(np.float64)
        for b in range(B):  # seeded rows of every sequence, all heads
            nb = int(lens[b])
            rows_i = np.unique(np.concatenate([rng.choice(nb, size=min(nb, 640), replace=False), [0, nb - 1]]))
            rows = np.stack([np.zeros(len(rows_i) * H, dtype=np.int64), np.repeat(np.arange(H), len(rows_i)),
                             np.tile(rows_i, H)], axis=1)
            sl = slice(int(cu[b]), int(cu[b + 1]))
            t_a = time.perf_counter()
            ob, lb = oracle.attention_rows_ex(qh[sl][None], kh[sl][None], vh[sl][None], dtype="bf16", layout="BSND",
                                              causal=True, scale=scale, rows=rows, nthreads=cores)
            t_cpu += time.perf_counter() - t_a
            n_rows += len(rows)
            sample_flops += float(np.sum(4.0 * D * (rows[:, 2] + 1)))
            got_o = o_h[int(cu[b]) + rows[:, 2], rows[:, 1]]
            got_l = l_h[rows[:, 1], int(cu[b]) + rows[:, 2]]
            err_o = max(err_o, float(np.abs(got_o - ob).max()))
            err_l = max(err_l, float(np.abs(got_l - lb).max()))
        cpu_tflops = sample_flops / t_cpu / 1e12
        cpu_baseline = {"value": round(cpu_tflops, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                        "sample": "%d seeded query rows over every sequence and head (%.3e FLOP, %.1f s); full-step "
                                  "time at this rate %.0f s" % (n_rows, sample_flops, t_cpu, flops / (cpu_tflops * 1e12))}
        parity = {"rows": n_rows, "max_abs_dO": err_o, "max_abs_dlse": err_l}
        log("bench: oracle %d rows in %.2f s; parity %s" % (n_rows, t_cpu, parity))
    line = {
        "metric": "attention fwd TFLOP/s, packed causal sequences of mixed length, H=32 D=128",
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
        "config": {"workload": "packed causal attention forward bf16, 8 sequences of lengths %s, H=%d D=%d"
                               % (list(map(int, lens)), H, D), "B": B, "H": H, "D": D, "total_tokens": total,
                   "max_seqlen": max_q, "causal": True, "scale": scale, "flop_per_step": flops},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline,
        "cpu_baseline": cpu_baseline,
        "parity_sample": parity,
    }
    finish_line(line, clocks)
    print(json.dumps(line), flush=True)


def bench_varlen_bwd(args):
    """One step = fa_bwd_varlen over the varlen workload's packed causal sequences; see the module notes."""
    import numpy as np
    import torch

    import transformer_attention_fwd_amd as fa
    from transformer_attention_fwd_amd import inputs

    B, H, D = 8, 32, 128
    lens = inputs.varlen_lengths(B, 512, 7680, seed=3)
    cu = inputs.cu_seqlens(lens)
    total = int(cu[-1])
    scale = float(np.float32(1.0 / np.sqrt(D)))
    log("bench: varlen lengths %s (total %d), backward" % (list(lens), total))
    qh, kh, vh = inputs.make_varlen(lens, lens, H, D, dtype="bf16", seed=3)
    doh = inputs.make_grad_varlen(lens, H, D, dtype="bf16", seed=3)
    to_dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda")
    q, k, v, do = to_dev(qh), to_dev(kh), to_dev(vh), to_dev(doh)
    cu_d = torch.from_numpy(cu).to("cuda")
    max_n = int(lens.max())
    o, lse = fa.attention_varlen(q, k, v, cu_d, cu_d, max_n, causal=True, scale=scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((H, total), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        st = fa.fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                              dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), cu_d.data_ptr(),
                              cu_d.data_ptr(), B, H, total, total, max_n, max_n, D, True, scale, fa.DTYPE_BF16,
                              stream.cuda_stream)
        if st != fa.FA_OK:
            raise RuntimeError("fa_bwd_varlen failed: %s %s" % (fa.status_str(st), fa.last_error()))

    log("bench: warmup %d" % args.warmup)
    args.steps = choose_steps(args, warmup_ms(step, args.warmup, torch))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    with ClockSampler() as clocks:
        t0 = time.perf_counter()
        for i in range(args.steps):
            ev[i][0].record(stream)
            step()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    call_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(args.steps)]
    ms_per_step = ev[0][0].elapsed_time(ev[-1][1]) / args.steps
    pairs = float(H * sum(int(n) * (int(n) + 1) // 2 for n in lens))
    flops = 10.0 * D * pairs
    value = flops / (ms_per_step * 1e-3) / 1e12
    mean_ms = float(np.mean(call_ms))
    achieved = flops / (mean_ms * 1e-3) / 1e12
    log("bench: %d steps, %.4f ms/step (wall %.4f), median %.4f ms, %.1f TFLOP/s"
        % (args.steps, ms_per_step, (t1 - t0) * 1e3 / args.steps, float(np.median(call_ms)), value))
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "kernel": "fa_bwd_dq<128,bf16,causal,varlen> + fa_bwd_dkdv<128,bf16,causal,varlen> (one fa_bwd_varlen "
                          "call)", "mean_launch_ms": round(mean_ms, 5), "launches_per_step": 2}
    cpu_baseline = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle

        cores = len(os.sched_getaffinity(0))  # the CPUs this process may use (the GPU machine: 16)
        rng = np.random.default_rng([4242, 3, 13])
        order = [divmod(int(x), H) for x in rng.permutation(B * H)]
        t_cpu, sample_flops, picked = 0.0, 0.0, []
        errs = {"dQ": 0.0, "dK": 0.0, "dV": 0.0}
        mags = {"dQ": 0.0, "dK": 0.0, "dV": 0.0}
        got_all = [t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv)]
        for b, h in order:  # seeded (sequence, head) pairs in full, until about 10 s of oracle time
            if t_cpu >= 10.0 and picked:
                break
            sl = slice(int(cu[b]), int(cu[b + 1]))
            t_a = time.perf_counter()
            ref = oracle.attention_bwd_ex(qh[sl][None], kh[sl][None], vh[sl][None], doh[sl][None], dtype="bf16",
                                          layout="BSND", causal=True, scale=scale, heads=[(0, h)], nthreads=cores)
            t_cpu += time.perf_counter() - t_a
            picked.append([b, h])
            nb = int(lens[b])
            sample_flops += 10.0 * D * nb * (nb + 1) / 2
            for name, g, r in zip(("dQ", "dK", "dV"), got_all, ref):
                errs[name] = max(errs[name], float(np.abs(g[sl, h] - r[0]).max()))
                mags[name] = max(mags[name], float(np.abs(r[0]).max()))
        cpu_tflops = sample_flops / t_cpu / 1e12
        cpu_baseline = {"value": round(cpu_tflops, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                        "sample": "%d whole (sequence, head) pairs of the same workload (dQ, dK, dV; %.3e FLOP, "
                                  "%.1f s); full-step time at this rate %.0f s"
                                  % (len(picked), sample_flops, t_cpu, flops / (cpu_tflops * 1e12))}
        parity = {"pairs": picked}
        for name in ("dQ", "dK", "dV"):
            parity["max_abs_err_" + name] = errs[name]
            parity["max_abs_ref_" + name] = mags[name]
        log("bench: oracle %d pairs in %.2f s; parity %s" % (len(picked), t_cpu, parity))
    line = {
        "metric": "attention bwd TFLOP/s (dQ, dK, dV), packed causal sequences of mixed length, H=32 D=128",
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
        "config": {"workload": "packed causal attention backward bf16, 8 sequences of lengths %s, H=%d D=%d"
                               % (list(map(int, lens)), H, D), "B": B, "H": H, "D": D, "total_tokens": total,
                   "max_seqlen": max_n, "causal": True, "scale": scale, "flop_per_step": flops},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline,
        "cpu_baseline": cpu_baseline,
        "parity_sample": parity,
    }
    finish_line(line, clocks)
    print(json.dumps(line), flush=True)


def bench_bwd(args, window=-1, dtype="bf16", atomic=False):
    """One step = fa_bwd (window < 0), fa_bwd_ex with that window, or fa_bwd_atomic over the C3 batch; see the
    module notes."""
    import numpy as np
    import torch

    import transformer_attention_fwd_amd as fa
    from transformer_attention_fwd_amd import inputs

    w = inputs.WORKLOADS["c3"]
    B, H, N, D = w.B, w.H, w.N, w.D
    log("bench: generating c3 inputs and dO %s" % ((B, H, N, D),))
    qh, kh, vh = inputs.make_workload(w, dtype)
    doh = inputs.make_grad(B, H, N, D, layout=w.layout, dtype=dtype, seed=w.seed)
    if dtype == "fp32":
        to_dev = lambda x: torch.from_numpy(x).to("cuda")
    else:
        to_dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda")
    dcode = fa.DTYPE_FP32 if dtype == "fp32" else fa.DTYPE_BF16
    peak = PEAK_FP32_TFLOPS if dtype == "fp32" else PEAK_BF16_TFLOPS
    q, k, v, do = to_dev(qh), to_dev(kh), to_dev(vh), to_dev(doh)
    o, lse = fa.attention_ex(q, k, v, layout=w.layout, causal=True, scale=w.scale, window=window)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    acc = torch.empty(q.shape, dtype=torch.float32, device="cuda") if atomic else None
    stream = torch.cuda.current_stream()
    layout = fa.LAYOUT_BHSD

    def step():
        if atomic:
            st = fa.fa_bwd_atomic(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                                  acc.data_ptr(), B, H, N, D, layout, True, w.scale, dcode, stream.cuda_stream)
        elif window < 0:
            st = fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                           dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B, H, N, D, layout, True,
                           w.scale, dcode, stream.cuda_stream)
        else:
            st = fa.fa_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                              do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B, H,
                              N, N, D, layout, True, window, 0, 0, N, w.scale, dcode, stream.cuda_stream)
        if st != fa.FA_OK:
            raise RuntimeError("fa_bwd failed: %s %s" % (fa.status_str(st), fa.last_error()))

    log("bench: warmup %d" % args.warmup)
    args.steps = choose_steps(args, warmup_ms(step, args.warmup, torch))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    with ClockSampler() as clocks:
        t0 = time.perf_counter()
        for i in range(args.steps):
            ev[i][0].record(stream)
            step()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    call_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(args.steps)]
    ms_per_step = ev[0][0].elapsed_time(ev[-1][1]) / args.steps
    pairs = float(B * H * visible_keys(N, N, 0, window).sum())
    flops = 10.0 * D * pairs
    value = flops / (ms_per_step * 1e-3) / 1e12
    mean_ms = float(np.mean(call_ms))
    achieved = flops / (mean_ms * 1e-3) / 1e12
    log("bench: %d steps, %.4f ms/step (wall %.4f), fa_bwd median %.4f ms best %.4f ms, %.1f TFLOP/s"
        % (args.steps, ms_per_step, (t1 - t0) * 1e3 / args.steps, float(np.median(call_ms)), min(call_ms), value))
    kern = ("fa_bwd_dq<128,bf16,causal> + fa_bwd_dkdv<128,bf16,causal> (one fa_bwd call)" if window < 0
            else "fa_bwd_dq<128,bf16,causal,window> + fa_bwd_dkdv<128,bf16,causal,window> (one fa_bwd_ex call)")
    if dtype == "fp32":
        kern = "fa_bwd_dq32<128,causal> + fa_bwd_dkdv32<128,causal> (one fa_bwd call)"
    if atomic:
        kern = ("fa_bwd_prep<128,bf16> + fa_bwd_dkdv<128,bf16,causal,atomic dQ> + fa_bwd_dq_convert<bf16> "
                "(one fa_bwd_atomic call)")
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": None, "kernel": kern,
                "mean_launch_ms": round(mean_ms, 5), "launches_per_step": 3 if atomic else 2}

    cpu_baseline = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle

        cores = len(os.sched_getaffinity(0))  # the CPUs this process may use (the GPU machine: 16)
        rng = np.random.default_rng([4242, 3, 9])
        order = [divmod(int(x), H) for x in rng.permutation(B * H)]
        heads, t_cpu, got, ref = [], 0.0, [], []
        while len(heads) < len(order) and (t_cpu < 10.0 or not heads):
            hd = order[len(heads)]
            t_a = time.perf_counter()
            r = oracle.attention_bwd_ex(qh, kh, vh, doh, dtype=dtype, layout=w.layout, causal=True, scale=w.scale,
                                        window=window, heads=[hd], nthreads=cores)
            t_cpu += time.perf_counter() - t_a
            heads.append(hd)
            ref.append([x[0] for x in r])
            got.append([t[hd[0], hd[1]].double().cpu().numpy() for t in (dq, dk, dv)])
        sample_flops = flops / (B * H) * len(heads)
        cpu_tflops = sample_flops / t_cpu / 1e12
        cpu_baseline = {"value": round(cpu_tflops, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                        "sample": "%d whole heads of the same workload (dQ, dK, dV; %.3e FLOP, %.1f s); full-step "
                                  "time at this rate %.0f s" % (len(heads), sample_flops, t_cpu,
                                                                 flops / (cpu_tflops * 1e12))}
        parity = {"heads": [list(h) for h in heads]}
        for n, name in enumerate(("dQ", "dK", "dV")):
            err = max(float(np.abs(g[n] - r_[n]).max()) for g, r_ in zip(got, ref))
            mag = max(float(np.abs(r_[n]).max()) for r_ in ref)
            parity["max_abs_err_" + name] = err
            parity["max_abs_ref_" + name] = mag
        log("bench: oracle %d heads in %.2f s on %d threads; parity %s" % (len(heads), t_cpu, cores, parity))

    line = {
        "metric": "attention bwd TFLOP/s (dQ, dK, dV), causal B=8 H=32 N=4096 D=128"
                  + ("" if window < 0 else ", window %d" % window) + ("" if dtype == "bf16" else ", " + dtype)
                  + (", atomic dQ" if atomic else ""),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": "causal attention backward %s B=%d H=%d N=%d D=%d %s%s%s"
                               % (dtype, B, H, N, D, w.layout, "" if window < 0 else " window %d" % window,
                                  " atomic dQ" if atomic else ""),
                   "B": B, "H": H, "N": N, "D": D, "layout": w.layout, "causal": True, "scale": w.scale,
                   "window": window, "flop_per_step": flops},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline,
        "cpu_baseline": cpu_baseline,
        "parity_sample": parity,
    }
    finish_line(line, clocks)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
