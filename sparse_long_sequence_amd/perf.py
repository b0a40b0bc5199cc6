"""Timing driver for the library's entry points on seeded synthetic inputs.

    python sparse_long_sequence_amd/perf.py attn  [--iters N] [--shape large|padded|long|tiny|large_fp32]
    python sparse_long_sequence_amd/perf.py attn_any [--iters N]  # same, 8 globals spread out
    python sparse_long_sequence_amd/perf.py prep  [--iters N]   # index compaction + mask shift
    python sparse_long_sequence_amd/perf.py layer [--iters N] [--dtype fp16|bf16|fp32]
    python sparse_long_sequence_amd/perf.py stack [--iters N] [--dtype fp16|bf16|fp32]
    python sparse_long_sequence_amd/perf.py ffn   [--iters N]   # FFN block, both paths
                                           # one encoder layer / the 24-layer encoder, B1 S1024
    python sparse_long_sequence_amd/perf.py table  # the five workloads: warm and cold time
    Any op: --calibrate-copy-mb N ends the run with one plain elementwise copy of N MiB
    (fp32 in, fp32 out), the known size HBM counters are scaled by.

Prints one JSON line per run: time per call (HIP events on the current stream around
N back-to-back calls after a warm-up) and the algorithmic throughput.  This is the
command profiles are taken with (rocprofv3 -- python3 <repo>/sparse_long_sequence_amd/perf.py
...); the headline benchmark is bench.py at the repository root.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import sparse_long_sequence_amd as lf  # noqa: E402
import workloads  # noqa: E402


WARMUP_SECONDS = 1.0   # --warmup-seconds


def _time(fn, iters: int, warmup: int) -> float:
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    # untimed calls (one second by default): the clocks ramp up over the first second
    # of work
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < WARMUP_SECONDS:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


ATTN_SHAPES = {"large": workloads.LARGE_FP16, "padded": workloads.PADDED_FP16,
               "long": workloads.LONG_BF16, "tiny": workloads.TINY_FP32,
               # the longformer-large shape in fp32 (vector-ALU attention)
               "large_fp32": workloads.AttnWorkload("longformer_large_fp32_B1_H16_S4096_W512_G8",
                                                    1, 16, 4096, 512, 8, "fp32", 20260002)}


def run_attn(iters: int, warmup: int, shape: str = "large") -> dict:
    wl = ATTN_SHAPES[shape]
    inp = workloads.make_attention_inputs(wl)
    g = {n: t.cuda() for n, t in inp.items()}
    out = torch.empty_like(g["q"])
    ms = _time(lambda: lf.attn_forward(g["q"], g["k"], g["v"], g["qg"], g["kg"], g["vg"],
                                       g["local_mask"], g["global_mask"], wl.W, wl.G, out=out),
               iters, warmup)
    # allowed pairs counted from the masks (padding excluded)
    flops = 256.0 * oracle_free_pairs(inp["local_mask"], inp["global_mask"], wl.W) * wl.H
    nbytes = sum(t.numel() * t.element_size() for t in inp.values()) + g["q"].numel() * g["q"].element_size()
    return {"op": "attn_forward", "workload": wl.name, "ms": ms,
            "tflops": flops / (ms * 1e-3) / 1e12, "alg_gbs": nbytes / (ms * 1e-3) / 1e9}


def run_attn_any(iters: int, warmup: int) -> dict:
    # the longformer-large shape with its 8 global tokens spread over the sequence
    # (tile edges, the middle, both ends) through lf_attn_forward_any_globals
    wl = workloads.LARGE_FP16
    pos = [[0, 255, 256, 1000, 2047, 2048, 3500, 4095]]
    inp = workloads.random_attention_inputs(wl.seed, wl.B, wl.H, wl.S, wl.W, wl.G, wl.dtype,
                                            global_positions=pos)
    g = {n: t.cuda() for n, t in inp.items()}
    out = torch.empty_like(g["q"])
    ms = _time(lambda: lf.attn_forward_any_globals(g["q"], g["k"], g["v"], g["qg"], g["kg"],
                                                   g["vg"], g["local_mask"], g["global_mask"],
                                                   wl.W, wl.G, out=out), iters, warmup)
    pairs = oracle_free_pairs(inp["local_mask"], inp["global_mask"], wl.W)
    flops = 256.0 * pairs * wl.H
    return {"op": "attn_forward_any_globals", "workload": wl.name + "_globals_spread",
            "ms": ms, "tflops": flops / (ms * 1e-3) / 1e12}


def oracle_free_pairs(local_mask, global_mask, W: int) -> int:
    """Allowed (query, key) pairs of one head, counted directly from the masks."""
    lm = (local_mask == 1).cpu().numpy()
    gl = (global_mask == 0).cpu().numpy()
    total = 0
    for b in range(lm.shape[0]):
        live, glob = lm[b], gl[b]
        S = live.shape[0]
        n_live, n_glob_live = int(live.sum()), int((live & glob).sum())
        band_ok = (live & ~glob).astype(np.int64)
        csum = np.concatenate([[0], np.cumsum(band_ok)])
        for s in range(S):
            if not live[s]:
                continue
            if glob[s]:
                total += n_live
            else:
                lo, hi = max(0, s - W // 2), min(S - 1, s + W // 2)
                total += n_glob_live + int(csum[hi + 1] - csum[lo])
    return total


def run_prep(iters: int, warmup: int) -> dict:
    wl = workloads.LONG_BF16
    inp = workloads.make_attention_inputs(wl)
    gm, lm = inp["global_mask"].cuda(), inp["local_mask"].cuda()
    B, S = gm.shape
    idx = torch.empty(B, S, dtype=torch.int32, device="cuda")
    cnt = torch.empty(B, dtype=torch.int32, device="cuda")
    bias = torch.empty_like(lm)
    ms_idx = _time(lambda: lf.init_global_idx(gm, idx, cnt), iters, warmup)
    ms_shift = _time(lambda: lf.mask_shift(lm, bias), iters, warmup)
    es = gm.element_size()
    idx_bytes = B * S * (es + 4) + B * 4
    shift_bytes = 2 * B * S * es
    # the headline masks (B=1, S=4096) as well
    wl1 = workloads.LARGE_FP16
    inp1 = workloads.make_attention_inputs(wl1)
    gm1 = inp1["global_mask"].cuda()
    idx1 = torch.empty(gm1.shape, dtype=torch.int32, device="cuda")
    cnt1 = torch.empty(gm1.shape[0], dtype=torch.int32, device="cuda")
    ms_idx1 = _time(lambda: lf.init_global_idx(gm1, idx1, cnt1), iters, warmup)
    return {"op": "prep", "workload": f"masks of {wl.name}", "ms_init_global_idx": ms_idx,
            "gbs_init_global_idx": idx_bytes / (ms_idx * 1e-3) / 1e9, "ms_mask_shift": ms_shift,
            "gbs_mask_shift": shift_bytes / (ms_shift * 1e-3) / 1e9,
            "ms_init_global_idx_" + wl1.name: ms_idx1}


def run_layer(iters: int, warmup: int, dtype: str = "fp16", any_globals: bool = False) -> dict:
    wl = workloads.LAYER_FP16
    t = workloads.make_layer_inputs(wl)
    td = workloads.TORCH_DTYPES[dtype]
    x = t["x"].cuda().to(td)
    w = {n: t[n].cuda().to(td) for n in lf.LAYER_WEIGHT_FIELDS}
    lm, gm = t["local_mask"].cuda().to(td), t["global_mask"].cuda().to(td)
    if any_globals:
        # the same number of global tokens, evenly spread over each sequence
        gm.fill_(workloads.NOT_GLOBAL)
        gm[:, torch.arange(wl.G, device="cuda") * (wl.S // wl.G) + wl.S // (2 * wl.G)] = 0.0
    y = torch.empty_like(x)
    nbytes = lf.encoder_layer_workspace_bytes(x.dtype, wl.B, wl.S, wl.hidden, wl.H, wl.ffn,
                                              wl.W, wl.G)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    ms = _time(lambda: lf.encoder_layer(x, w, lm, gm, wl.H, wl.W, wl.G, out=y, workspace=ws,
                                        any_globals=any_globals), iters, warmup)
    M, D, F, G, S, W = wl.B * wl.S, wl.hidden, wl.ffn, wl.G, wl.S, wl.W
    gemm = 2.0 * M * D * (5 * D + D + 2 * F) + 2.0 * wl.B * G * D * D
    pairs = G * S + (S - G) * (W + 1 + G) - (W // 2) * (W // 2 + 1)
    attn = 256.0 * pairs * wl.B * wl.H
    name = wl.name.replace("fp16", dtype) + ("_globals_spread" if any_globals else "")
    return {"op": "encoder_layer" + ("_any_globals" if any_globals else ""), "workload": name,
            "ms": ms,
            "gemm_gflop": gemm / 1e9, "attn_gflop": attn / 1e9,
            "tflops": (gemm + attn) / (ms * 1e-3) / 1e12}


def run_stack(iters: int, warmup: int, dtype: str = "fp16", n_layers: int = 24) -> dict:
    # the pages' benchmark model: 16 heads x 64, FFN 4096, window 512, 24 layers, at
    # batch 1 and sequence 1024; 16 leading global tokens (the count is not stated)
    B, S, D, H, F, W, G = 1, 1024, 1024, 16, 4096, 512, 16
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20260006)
    dt = workloads.TORCH_DTYPES[dtype]

    def rnd(*shape, std=0.02):
        return (torch.randn(*shape, generator=gen, device="cuda") * std).to(dt)

    layers = []
    for _ in range(n_layers):
        w = {"w_proj": rnd(5 * D, D), "w_qg": rnd(D, D), "w_o": rnd(D, D),
             "w_ffn1": rnd(F, D), "w_ffn2": rnd(D, F)}
        for n, size in (("b_proj", 5 * D), ("b_qg", D), ("b_o", D), ("b_ffn1", F), ("b_ffn2", D)):
            w[n] = torch.zeros(size, dtype=dt, device="cuda")
        for n in ("ln1", "ln2"):
            w[n + "_g"] = torch.ones(D, dtype=dt, device="cuda")
            w[n + "_b"] = torch.zeros(D, dtype=dt, device="cuda")
        layers.append(w)
    x = torch.randn(B, S, D, generator=gen, device="cuda").to(dt)
    lm = torch.ones(B, S, dtype=dt, device="cuda")
    gm = torch.full((B, S), -10000.0, dtype=dt, device="cuda")
    gm[:, :G] = 0.0
    y = torch.empty_like(x)
    nbytes = lf.encoder_forward_workspace_bytes(dt, B, S, D, H, F, W, G)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    ms = _time(lambda: lf.encoder_forward(x, layers, lm, gm, H, W, G, out=y, workspace=ws),
               iters, warmup)
    M = B * S
    gemm = 2.0 * M * D * (5 * D + D + 2 * F) + 2.0 * B * G * D * D
    pairs = G * S + (S - G) * (W + 1 + G) - (W // 2) * (W // 2 + 1)
    attn = 256.0 * pairs * B * H
    return {"op": "encoder_forward", "workload": f"longformer_large_24L_{dtype}_B{B}_S{S}_W{W}_G{G}",
            "layers": n_layers, "ms": ms, "ms_per_layer": ms / n_layers,
            "tflops": n_layers * (gemm + attn) / (ms * 1e-3) / 1e12}


def run_ffn(iters: int, warmup: int, dtype: str = "fp16") -> dict:
    # the FFN block (step 6) at the layer's rows (B 2 x S 4096) and at the stack
    # benchmark's (B 1 x S 1024), D 1024, F 4096, both paths
    D, F = 1024, 4096
    td = workloads.TORCH_DTYPES[dtype]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20260007)
    w1 = (torch.randn(F, D, generator=gen, device="cuda") * 0.02).to(td)
    w2 = (torch.randn(D, F, generator=gen, device="cuda") * 0.02).to(td)
    b1 = torch.zeros(F, dtype=td, device="cuda")
    b2, beta = (torch.zeros(D, dtype=td, device="cuda") for _ in range(2))
    gamma = torch.ones(D, dtype=td, device="cuda")
    res = {"op": "ffn_block", "dtype": dtype, "D": D, "F": F}
    for M in (8192, 1024):
        resid = torch.randn(M, D, generator=gen, device="cuda")
        h = resid.to(td)
        y = torch.empty_like(h)
        flop = 4.0 * M * D * F
        for fused in (False, True):
            nb = lf.ffn_block_workspace_bytes(td, M, D, F, fused)
            ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
            ms = _time(lambda: lf.ffn_block(h, resid, w1, b1, w2, b2, gamma, beta, fused,
                                            out=y, workspace=ws), iters, warmup)
            key = f"M{M}_{'fused' if fused else 'two_gemm'}"
            res[key + "_ms"] = ms
            res[key + "_tflops"] = flop / (ms * 1e-3) / 1e12
    return res


def _time_trials(fn, trials: int, calls: int) -> float:
    """Median over `trials` of the per-call time of `calls` back-to-back calls (after a
    second of untimed calls, so the clocks have ramped up)."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 1.0:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    res = []
    for _ in range(trials):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(calls):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) / calls)
    return sorted(res)[len(res) // 2]


def _time_cold(fn, calls: int) -> float:
    """Median time of `calls` single calls, each enqueued right after a 512 MiB fill that
    evicts L2 and the Infinity Cache (the interval holds only the call)."""
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    res = []
    for i in range(calls):
        scrub.fill_(i & 0xff)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1))
    del scrub
    return sorted(res)[len(res) // 2]


PEAK = {"fp16": 2516.6, "bf16": 2516.6, "fp32": 157.3}   # dense MFMA TFLOP/s (fp32: FMA)


def run_table() -> list:
    """The five workloads (tiny fp32, longformer-large fp16, padded fp16, long bf16, the
    fp16 encoder layer): warm time (median of 5 trials of back-to-back calls), cold time
    (median of 20 calls after a cache scrub), algorithmic TFLOP/s and GB/s."""
    out = []
    for wl in workloads.ATTN_WORKLOADS:
        inp = workloads.make_attention_inputs(wl)
        g = {n: t.cuda() for n, t in inp.items()}
        o = torch.empty_like(g["q"])
        fn = lambda: lf.attn_forward(g["q"], g["k"], g["v"], g["qg"], g["kg"], g["vg"],
                                     g["local_mask"], g["global_mask"], wl.W, wl.G, out=o)
        warm = _time_trials(fn, 5, 200)
        cold = _time_cold(fn, 20)
        flops = 256.0 * oracle_free_pairs(inp["local_mask"], inp["global_mask"], wl.W) * wl.H
        nbytes = sum(t.numel() * t.element_size() for t in inp.values()) + o.numel() * o.element_size()
        out.append({"workload": wl.name, "ms_warm": warm, "ms_cold": cold,
                    "tflops": flops / (warm * 1e-3) / 1e12,
                    "pct_peak": 100.0 * flops / (warm * 1e-3) / 1e12 / PEAK[wl.dtype],
                    "peak_tflops": PEAK[wl.dtype], "alg_gbs": nbytes / (warm * 1e-3) / 1e9,
                    "alg_bytes": nbytes, "alg_gflop": flops / 1e9})
        del g, o
    wl = workloads.LAYER_FP16
    t = workloads.make_layer_inputs(wl)
    x = t["x"].cuda()
    w = {n: t[n].cuda() for n in lf.LAYER_WEIGHT_FIELDS}
    lm, gm = t["local_mask"].cuda(), t["global_mask"].cuda()
    y = torch.empty_like(x)
    nb = lf.encoder_layer_workspace_bytes(x.dtype, wl.B, wl.S, wl.hidden, wl.H, wl.ffn, wl.W, wl.G)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    fn = lambda: lf.encoder_layer(x, w, lm, gm, wl.H, wl.W, wl.G, out=y, workspace=ws)
    warm = _time_trials(fn, 5, 20)
    cold = _time_cold(fn, 20)
    M, D, F, G, S, W = wl.B * wl.S, wl.hidden, wl.ffn, wl.G, wl.S, wl.W
    gemm = 2.0 * M * D * (5 * D + D + 2 * F) + 2.0 * wl.B * G * D * D
    pairs = G * S + (S - G) * (W + 1 + G) - (W // 2) * (W // 2 + 1)
    flops = gemm + 256.0 * pairs * wl.B * wl.H
    out.append({"workload": wl.name, "ms_warm": warm, "ms_cold": cold,
                "tflops": flops / (warm * 1e-3) / 1e12,
                "pct_peak": 100.0 * flops / (warm * 1e-3) / 1e12 / PEAK["fp16"],
                "peak_tflops": PEAK["fp16"], "alg_gflop": flops / 1e9})
    return out


def calibrate_copy(mib: int):
    """One plain elementwise copy of `mib` MiB (fp32 read, fp32 written)."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("op", choices=["attn", "attn_any", "prep", "layer", "stack", "ffn", "table"])
    ap.add_argument("--iters", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--dtype", default="fp16", choices=["fp16", "bf16", "fp32"],
                    help="layer / stack only")
    ap.add_argument("--shape", default="large", choices=sorted(ATTN_SHAPES),
                    help="attn only: longformer-large, padded (B4 H12 G32) or long (bf16 S16384)")
    ap.add_argument("--any-globals", action="store_true",
                    help="layer only: globals spread over the sequence, general entry point")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="end with one plain elementwise copy of this many MiB (counter scaling)")
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="untimed calls before timing (0 under a counter profiler)")
    a = ap.parse_args()
    global WARMUP_SECONDS
    WARMUP_SECONDS = a.warmup_seconds
    if a.op == "layer":
        print(json.dumps(run_layer(a.iters, a.warmup, a.dtype, a.any_globals)), flush=True)
    elif a.op == "stack":
        print(json.dumps(run_stack(a.iters, a.warmup, a.dtype)), flush=True)
    elif a.op == "ffn":
        print(json.dumps(run_ffn(a.iters, a.warmup, a.dtype)), flush=True)
    elif a.op == "attn":
        print(json.dumps(run_attn(a.iters, a.warmup, a.shape)), flush=True)
    elif a.op == "table":
        for r in run_table():
            print(json.dumps(r), flush=True)
    else:
        fn = {"attn_any": run_attn_any, "prep": run_prep}[a.op]
        print(json.dumps(fn(a.iters, a.warmup)), flush=True)
    if a.calibrate_copy_mb > 0:
        calibrate_copy(a.calibrate_copy_mb)


if __name__ == "__main__":
    main()
