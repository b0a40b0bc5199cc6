"""Seeded synthetic inputs for the Longformer band + global attention workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  Both the GPU tests / bench and the CPU oracle consume what
it produces, so the two sides always see bit-identical inputs.

Shapes follow the longformer-large encoder the FasterTransformer Longformer page
benchmarks (section "性能基准：FP32 与 FP16": 16 heads x 64, intermediate 4096,
local window 512).  No checkpoint or dataset is used: every tensor is drawn from
a seeded ``numpy.random.default_rng`` and rounded to the activation dtype with
round-to-nearest-even; the rounded tensor is the canonical input for both sides.

Mask encodings follow the page's input list in section "Longformer Encoder
计算流程": local mask 1.0 = attends, 0.0 = padding; global mask 0.0 = global
token, -10000.0 = ordinary token.  Global tokens sit contiguously at the head of
each sequence (the page's fourth hard constraint), unless explicit per-sequence
positions are given (the globals-anywhere entry point).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

HEAD_DIM = 64
NOT_GLOBAL = -10000.0

TORCH_DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class AttnWorkload:
    """One attention workload: q,k,v,kg,vg,out are [B,H,S,64]; qg is [B,H,G,64]."""
    name: str
    B: int
    H: int
    S: int
    W: int
    G: int
    dtype: str
    seed: int
    std: float = 0.125
    pad_frac: tuple | None = None   # (lo, hi): per sequence a trailing U[lo,hi] share is padding
    n_global: tuple | None = None   # per-batch global count; default G for every sequence
    global_positions: tuple | None = None   # per-batch position tuples (overrides n_global)


@dataclass(frozen=True)
class LayerWorkload:
    """One encoder layer: x is [B,S,hidden], weights use the [out,in] row-major layout."""
    name: str
    B: int
    S: int
    hidden: int
    H: int
    ffn: int
    W: int
    G: int
    dtype: str
    seed: int
    w_std: float = 0.02
    extra: dict = field(default_factory=dict)


# The five measured / parity workloads.  Seeds are 20260000 + workload number.
TINY_FP32 = AttnWorkload("tiny_fp32_B1_H2_S64_W16_G2", 1, 2, 64, 16, 2, "fp32", 20260001)
LARGE_FP16 = AttnWorkload("longformer_large_fp16_B1_H16_S4096_W512_G8", 1, 16, 4096, 512, 8,
                          "fp16", 20260002)
PADDED_FP16 = AttnWorkload("padded_fp16_B4_H12_S4096_W512_G32", 4, 12, 4096, 512, 32, "fp16",
                           20260003, pad_frac=(0.10, 0.25))
LONG_BF16 = AttnWorkload("long_bf16_B2_H16_S16384_W512_G64", 2, 16, 16384, 512, 64, "bf16",
                         20260004)
LAYER_FP16 = LayerWorkload("encoder_layer_fp16_B2_S4096_D1024_H16_F4096_W512_G16", 2, 4096,
                           1024, 16, 4096, 512, 16, "fp16", 20260005)

ATTN_WORKLOADS = [TINY_FP32, LARGE_FP16, PADDED_FP16, LONG_BF16]


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(TORCH_DTYPES[dtype])


def make_masks(rng: np.random.Generator, B: int, S: int, G: int, dtype: str,
               pad_frac=None, n_global=None, global_positions=None):
    """Local mask (1 = token, 0 = padding) and global mask (0 = global, -10000 = not).

    Global tokens: positions 0 .. n-1 of each sequence (n = n_global[b], default G),
    or, when ``global_positions`` is given, exactly ``global_positions[b]``.
    """
    local = np.ones((B, S), np.float64)
    glob = np.full((B, S), NOT_GLOBAL, np.float64)
    counts = list(n_global) if n_global is not None else [G] * B
    for b in range(B):
        if global_positions is not None:
            glob[b, list(global_positions[b])] = 0.0
        else:
            glob[b, : counts[b]] = 0.0
    if pad_frac is not None:
        lo, hi = pad_frac
        for b in range(B):
            f = rng.uniform(lo, hi)
            pad = int(round(f * S))
            if pad > 0:
                local[b, S - pad:] = 0.0
    return _cast(local, dtype), _cast(glob, dtype)


def make_attention_inputs(wl: AttnWorkload, std: float | None = None) -> dict:
    """CPU tensors q,k,v,qg,kg,vg,local_mask,global_mask in ``wl.dtype``.

    Draw order is fixed: q, k, v, qg, kg, vg, then the padding fractions.
    """
    rng = np.random.default_rng(wl.seed)
    s = wl.std if std is None else std
    B, H, S, G, D = wl.B, wl.H, wl.S, wl.G, HEAD_DIM
    out = {}
    for name, rows in (("q", S), ("k", S), ("v", S), ("qg", G), ("kg", S), ("vg", S)):
        out[name] = _cast(rng.standard_normal((B, H, rows, D)) * s, wl.dtype)
    out["local_mask"], out["global_mask"] = make_masks(
        rng, B, S, G, wl.dtype, wl.pad_frac, wl.n_global, wl.global_positions)
    return out


def make_layer_inputs(wl: LayerWorkload) -> dict:
    """CPU tensors for one encoder layer.

    x ~ N(0,1); weights ~ N(0, w_std^2) drawn in the order proj, qg, o, ffn1, ffn2;
    biases zero; LayerNorm gamma = 1, beta = 0.  Weights are [out, in] row-major;
    ``w_proj`` stacks the Q, K, V, global-K, global-V blocks along its rows.
    """
    rng = np.random.default_rng(wl.seed)
    D, F = wl.hidden, wl.ffn
    t = {}
    t["x"] = _cast(rng.standard_normal((wl.B, wl.S, D)), wl.dtype)
    t["w_proj"] = _cast(rng.standard_normal((5 * D, D)) * wl.w_std, wl.dtype)
    t["w_qg"] = _cast(rng.standard_normal((D, D)) * wl.w_std, wl.dtype)
    t["w_o"] = _cast(rng.standard_normal((D, D)) * wl.w_std, wl.dtype)
    t["w_ffn1"] = _cast(rng.standard_normal((F, D)) * wl.w_std, wl.dtype)
    t["w_ffn2"] = _cast(rng.standard_normal((D, F)) * wl.w_std, wl.dtype)
    t["b_proj"] = _cast(np.zeros(5 * D), wl.dtype)
    t["b_qg"] = _cast(np.zeros(D), wl.dtype)
    t["b_o"] = _cast(np.zeros(D), wl.dtype)
    t["b_ffn1"] = _cast(np.zeros(F), wl.dtype)
    t["b_ffn2"] = _cast(np.zeros(D), wl.dtype)
    t["ln1_g"] = _cast(np.ones(D), wl.dtype)
    t["ln1_b"] = _cast(np.zeros(D), wl.dtype)
    t["ln2_g"] = _cast(np.ones(D), wl.dtype)
    t["ln2_b"] = _cast(np.zeros(D), wl.dtype)
    t["local_mask"], t["global_mask"] = make_masks(rng, wl.B, wl.S, wl.G, wl.dtype)
    return t


def random_layer_params(rng: np.random.Generator, D: int, F: int, dtype: str,
                        w_std: float = 0.02, b_std: float = 0.0, ln_jitter: float = 0.0) -> dict:
    """Layer parameters with optional non-trivial biases / LayerNorm affine terms."""
    t = {}
    shapes = {"w_proj": (5 * D, D), "w_qg": (D, D), "w_o": (D, D),
              "w_ffn1": (F, D), "w_ffn2": (D, F)}
    for n, shp in shapes.items():
        t[n] = _cast(rng.standard_normal(shp) * w_std, dtype)
    for n, size in (("b_proj", 5 * D), ("b_qg", D), ("b_o", D), ("b_ffn1", F), ("b_ffn2", D)):
        t[n] = _cast(rng.standard_normal(size) * b_std, dtype)
    for n in ("ln1", "ln2"):
        t[n + "_g"] = _cast(1.0 + rng.standard_normal(D) * ln_jitter, dtype)
        t[n + "_b"] = _cast(rng.standard_normal(D) * ln_jitter, dtype)
    return t


def random_attention_inputs(seed: int, B: int, H: int, S: int, W: int, G: int, dtype: str,
                            std: float = 0.125, pad_frac=None, n_global=None,
                            global_positions=None) -> dict:
    """Same recipe as ``make_attention_inputs`` for an ad-hoc shape."""
    gp = tuple(tuple(int(x) for x in p) for p in global_positions) if global_positions is not None \
        else None
    wl = AttnWorkload("adhoc", B, H, S, W, G, dtype, seed, std, pad_frac,
                      tuple(n_global) if n_global is not None else None, gp)
    return make_attention_inputs(wl)
