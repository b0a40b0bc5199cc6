#!/usr/bin/env python3
"""Benchmark of Longformer band + global attention on one MI355X.

Workload: the longformer-large-shaped problem (B=1, H=16 heads x 64, S=4096,
window W=512 i.e. +-256, G=8 leading global tokens, fp16), seeded synthetic
inputs already resident in HBM.  One step = one lf_attn_forward call on the raw
masks: one kernel launch that counts the leading global tokens from the global mask
and tests keys against the local mask where it uses them (so the separate index and
mask-shift kernels of the preprocessing entry points do not run), then the band and
global-key scores, the masked online softmax, PV, the global rows and the output.

Prints ONE JSON line on stdout.  After W warm-up steps and `--warmup-seconds` of
further untimed steps (the GPU clocks ramp up over the first second of work), K
steps are timed between two events: `value` is effective TFLOP/s = algorithmic
flops (256 per allowed (query, key) pair) / time per step.  A step is one launch of
the band + global-row kernel, so the same events give that kernel's average launch
duration.  `roofline` reports that kernel against the roofline that
binds at its algorithmic intensity (flops / algorithmic bytes vs the ridge point
2516.6 TFLOP/s / 8 TB/s); the MFMA fraction is reported beside it.  `traffic` is
the counter-measured HBM bytes per launch from the committed summary, when it was
taken on the current kernel sources.  `cpu_baseline` times the float64 oracle on a
bounded sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "band+global attention ms and TFLOP/s (% MFMA peak), B=1 H=16 S=4096 W=512 fp16"
PEAK_FP16_TFLOPS = 2516.6        # MI355X dense fp16 MFMA: 256 CU x 4 SIMD x 1024 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
LAUNCHES_PER_STEP = 1            # lf_attn_forward on fp16 / bf16 inputs: one kernel launch
KERNEL_SOURCES = ["sparse_long_sequence_amd/csrc/attn_mfma.hip",
                  "sparse_long_sequence_amd/csrc/attn_mfma_gwg.hip",
                  "sparse_long_sequence_amd/csrc/lf_device.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_mfma_longformer_large_fp16_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def pairs_per_head(S: int, W: int, G: int) -> int:
    """Allowed (query, key) pairs of one unpadded head with G leading global tokens."""
    return G * S + (S - G) * (W + 1 + G) - (W // 2) * (W // 2 + 1)


def row_pairs(s: int, S: int, W: int, G: int) -> int:
    if s < G:
        return S
    lo, hi = max(G, s - W // 2), min(S - 1, s + W // 2)
    return G + (hi - lo + 1)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic():
    """Per-launch HBM bytes of the dominant kernel from the committed counter summary,
    or None when it is absent or was taken on different kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    txt = open(TRAFFIC_FILE).read()
    m_src = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not (m_src and m_b) or m_src.group(1) != kernel_source_hash():
        return None
    return float(m_b.group(1))


def cpu_baseline(inp, wl, budget_s: float):
    """Time the float64 oracle on rows of the workload until the budget is spent, with
    its BLAS using every core this process may run on; returns throughput in the
    metric's unit (TFLOP/s)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    cores = len(os.sched_getaffinity(0))
    rows, flops, t_total, passes = 0, 0.0, 0.0, 0
    with threadpool_limits(limits=cores):
        blas = ",".join(sorted({f"{i.get('internal_api')} {i.get('version')} x{i.get('num_threads')}"
                                for i in threadpool_info() if i.get("user_api") == "blas"}))
        # whole heads of batch 0 in blocks of 256 rows, head after head, starting
        # over at head 0 until the time budget is spent
        while t_total < budget_s:
            h = (rows // wl.S) % wl.H
            for s0 in range(0, wl.S, 256):
                rr = [(0, h, s) for s in range(s0, min(wl.S, s0 + 256))]
                t0 = time.perf_counter()
                oracle.attention(inp["q"], inp["k"], inp["v"], inp["qg"], inp["kg"], inp["vg"],
                                 inp["local_mask"], inp["global_mask"], wl.W, wl.G, rows=rr)
                t_total += time.perf_counter() - t0
                rows += len(rr)
                flops += 256.0 * sum(row_pairs(s, wl.S, wl.W, wl.G) for (_, _, s) in rr)
            passes = rows / (wl.H * wl.S)
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows} query rows ({passes:.2f} passes over the {wl.H} x {wl.S} rows of "
                      f"batch 0) of the same workload, whole heads of {wl.S} rows, "
                      f"{t_total:.1f} s of float64 numpy oracle time, BLAS threads = {cores} "
                      f"(the process's CPU affinity; the oracle's per-row products are small, "
                      f"so most of its time is single-threaded Python)",
            "blas": blas, "seconds": round(t_total, 2), "host_cpus": os.cpu_count()}


def oracle_table():
    """The float64 oracle over the whole output of each graded configuration (the same
    calls the full-output parity tests make), BLAS threads = this process's CPU
    affinity; one JSON line per configuration.  CPU only: no GPU work."""
    from threadpoolctl import threadpool_limits

    import oracle
    import workloads
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        for wl in workloads.ATTN_WORKLOADS:
            inp = workloads.make_attention_inputs(wl)
            t0 = time.perf_counter()
            oracle.attention(inp["q"], inp["k"], inp["v"], inp["qg"], inp["kg"], inp["vg"],
                             inp["local_mask"], inp["global_mask"], wl.W, wl.G)
            dt = time.perf_counter() - t0
            print(json.dumps({"workload": wl.name, "oracle_s": round(dt, 3), "cores": cores,
                              "rows": wl.B * wl.H * wl.S}), flush=True)
        wl = workloads.LAYER_FP16
        t = workloads.make_layer_inputs(wl)
        w = {n: t[n] for n in ["w_proj", "b_proj", "w_qg", "b_qg", "w_o", "b_o", "ln1_g", "ln1_b",
                               "w_ffn1", "b_ffn1", "w_ffn2", "b_ffn2", "ln2_g", "ln2_b"]}
        t0 = time.perf_counter()
        oracle.encoder_layer(t["x"], w, t["local_mask"], t["global_mask"], wl.H, wl.W, wl.G)
        dt = time.perf_counter() - t0
        print(json.dumps({"workload": wl.name, "oracle_s": round(dt, 3), "cores": cores,
                          "rows": wl.B * wl.S}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="after the W warm-up steps, keep launching untimed steps for this long "
                         "so the GPU clocks have ramped up before anything is timed")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the oracle CPU baseline (0 = skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--trials", type=int, default=5,
                    help="after the K timed steps, this many further trials of --trial-steps "
                         "steps each; their median per-step time is reported beside the value")
    ap.add_argument("--trial-steps", type=int, default=200)
    ap.add_argument("--cold-calls", type=int, default=20,
                    help="after the timed steps, time this many single steps each right after "
                         "a 512 MiB scrub write (caches cold; reported beside the value)")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="after the timed loop, run one plain elementwise copy of this many MiB "
                         "(fp32 in, fp32 out) so HBM counters can be scaled by a known size")
    ap.add_argument("--oracle-table", action="store_true",
                    help="only time the float64 oracle over the whole output of each graded "
                         "configuration on this host's cores (CPU only), one JSON line each")
    args = ap.parse_args()
    if args.oracle_table:
        oracle_table()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested). The (batch, head) pairs of the attention are "
              f"independent, so they would shard across GPUs with no communication.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_long_sequence_amd as lf
    import workloads

    wl = workloads.LARGE_FP16
    inp = workloads.make_attention_inputs(wl)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = {n: t.to(dev) for n, t in inp.items()}
    out = torch.empty_like(g["q"])

    def step():
        lf.attn_forward(g["q"], g["k"], g["v"], g["qg"], g["kg"], g["vg"], g["local_mask"],
                        g["global_mask"], wl.W, wl.G, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < args.warmup_seconds:
        for _ in range(100):
            step()
        torch.cuda.synchronize()
    # K steps between two events recorded on the stream the kernel is launched on
    # (torch's current stream, which the binding passes to the library).  A step is
    # exactly one kernel launch, so (end - start) / K is also the kernel's average
    # launch duration (gaps between back-to-back launches included).  Events around
    # every launch would add several microseconds per launch, so there are none.
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    n_k, k_ms = args.steps * LAUNCHES_PER_STEP, e0.elapsed_time(e1)
    # secondary: 5 trials of 200 back-to-back steps, median per-step time
    trial_ms = []
    for _ in range(args.trials):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(args.trial_steps):
            step()
        t1.record()
        torch.cuda.synchronize()
        trial_ms.append(t0.elapsed_time(t1) / args.trial_steps)
    trials = None
    if trial_ms:
        srt = sorted(trial_ms)
        trials = {"n_trials": len(srt), "steps_per_trial": args.trial_steps,
                  "ms_per_step_median": round(srt[len(srt) // 2], 6),
                  "ms_per_step_min": round(srt[0], 6), "ms_per_step_max": round(srt[-1], 6)}
    # secondary: cold caches.  A 512 MiB fill evicts L2 and the 256 MiB Infinity Cache;
    # the events and the step are enqueued while the fill still runs, so the interval
    # holds only the step.
    cold = None
    if args.cold_calls > 0:
        scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        times = []
        for i in range(args.cold_calls):
            scrub.fill_(i & 0xff)
            c0 = torch.cuda.Event(enable_timing=True)
            c1 = torch.cuda.Event(enable_timing=True)
            c0.record()
            step()
            c1.record()
            torch.cuda.synchronize()
            times.append(c0.elapsed_time(c1))
        del scrub
        times.sort()
        cold = {"ms_per_step_median": round(times[len(times) // 2], 6),
                "ms_per_step_min": round(times[0], 6), "calls": args.cold_calls,
                "scrub_mib": 512}
    if args.calibrate_copy_mb > 0:
        n = args.calibrate_copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)   # reads and writes calibrate_copy_mb MiB each
        torch.cuda.synchronize()
        log(f"calibration copy: {args.calibrate_copy_mb} MiB read + {args.calibrate_copy_mb} MiB written")
    k_avg_ms = k_ms / n_k

    flops = 256.0 * pairs_per_head(wl.S, wl.W, wl.G) * wl.B * wl.H
    tflops = flops / (ms * 1e-3) / 1e12
    k_tflops = flops / (k_avg_ms * 1e-3) / 1e12
    alg_bytes = 2 * (6 * wl.B * wl.H * wl.S * 64 + wl.B * wl.H * wl.G * 64 + 2 * wl.B * wl.S)
    log(f"step {ms * 1e3:.2f} us, main kernel {k_avg_ms * 1e3:.2f} us over {n_k} launches, "
        f"{tflops:.1f} TFLOP/s step, {k_tflops:.1f} TFLOP/s kernel, "
        f"{alg_bytes / (k_avg_ms * 1e-3) / 1e9:.0f} GB/s algorithmic")

    traffic = stored_traffic()
    # which roofline binds: algorithmic intensity against the ridge point
    ridge = PEAK_FP16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    intensity = flops / alg_bytes
    hbm_gbs = alg_bytes / (k_avg_ms * 1e-3) / 1e9
    if intensity < ridge:
        roof = {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(hbm_gbs / PEAK_HBM_GBS, 5)}
    else:
        roof = {"bound": "mfma", "achieved": round(k_tflops, 3), "peak": PEAK_FP16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(k_tflops / PEAK_FP16_TFLOPS, 5)}
    roof.update({
        "traffic": traffic,
        "kernel": "attn_mfma_kernel (band tiles + global-row splits)",
        "kernel_avg_us": round(k_avg_ms * 1e3, 3),
        "algorithmic_flops_per_launch": flops,
        "algorithmic_bytes_per_launch": alg_bytes,
        "intensity_flop_per_byte": round(intensity, 1),
        "ridge_flop_per_byte": round(ridge, 1),
        "mfma_achieved_tflops": round(k_tflops, 3),
        "mfma_frac": round(k_tflops / PEAK_FP16_TFLOPS, 5),
    })
    res = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_seconds": args.warmup_seconds,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "S": wl.S, "W": wl.W, "G": wl.G,
                   "head_dim": 64},
        "pct_mfma_peak": round(100.0 * tflops / PEAK_FP16_TFLOPS, 3),
        "roofline": roof,
    }
    if trials is not None:
        res["trials"] = trials
    if cold is not None:
        res["cold_cache"] = cold
    if not args.no_cpu_baseline and args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(inp, wl, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
