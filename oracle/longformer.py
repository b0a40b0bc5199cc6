"""Float64 CPU oracle for Longformer local sliding-window + global attention.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library (no kernels, headers, tables or helpers) and never imports
it; the only thing both sides share is the seeded input generator in
``workloads``.

What it follows.  The page "FasterTransformer Longformer 推理加速实践：PyTorch
集成、输入约束与端到端性能解析" (cited as [FT-LF]):
  * section "Longformer Encoder 计算流程" (encoder computation flow), its input
    list (mask encodings), its preprocessing list (global-index extraction and
    the local-mask shift) and its per-layer steps 1-6;
  * section "使用前提：四条硬性约束" (the four hard constraints).

The method computes exactly the masked-softmax attention, so each attention
function below is that definition written out row by row; the layer is the
page's per-layer step list in order.  Inputs arrive already rounded to the
activation dtype and are widened exactly to float64; nothing else is rounded,
except the mask-shift output, whose precision the page fixes (an fp32 fma).

Readings taken where the page is silent or loose (all in the docstrings below):
  R1 band endpoints: a local row s sees keys j with |j - s| <= W/2 (W+1 keys);
  R2 the band is truncated at the sequence ends (no wrap-around);
  R3 global positions are removed from the band and counted once, as global keys;
  R4 local rows read k, v at global positions; kg, vg, qg serve global rows only;
  R5 score scale is a parameter, 1/sqrt(64) = 0.125 by default;
  R6 a padded key (local mask 0) is excluded from every row, global rows included;
  R7 a padded row (local mask 0) is exactly +0.0, global or not;
  R8 a token is global iff its global-mask value equals 0.0;
  R9 the index buffer is a full stable partition: flagged positions ascending,
     then the unflagged ones in descending order;
  R10 qg holds G rows; row r belongs to the r-th global position;
  R11 LayerNorm: biased variance, eps 1e-5; GELU is the exact erf form; no dropout.

Pins (tests/test_oracle_pins.py): hand-derived fixtures under tests/golden/, a
dense boolean-mask brute force through torch's scaled-dot-product attention,
row-sum, closed-form (q = 0 gives the mean of the allowed v rows; v = I reads
out the probabilities), full-attention reductions, exact zero for padded rows,
textbook GELU values and LayerNorm moments.  No function here is "parity
unpinned".
"""
from __future__ import annotations

import math

import numpy as np
import torch
from scipy.special import erf

_TORCH = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


def _f64(x) -> np.ndarray:
    """Exact widening of a tensor / array (fp16, bf16, fp32, fp64) to float64."""
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# [FT-LF "Longformer Encoder 计算流程", preprocessing, first item]: per batch row,
# extract the positions of the global tokens and their count from the global
# mask with a flagged partition.
# ---------------------------------------------------------------------------
def global_partition(global_mask):
    """Return (global_idx int32 [B,S], global_count int32 [B]).

    R8: position s is flagged iff global_mask[b,s] == 0.0 (-0.0 counts as 0.0).
    R9: global_idx[b] lists the flagged positions in ascending order, followed
    by the remaining positions in descending order, so each row is a
    permutation of 0..S-1; global_count[b] is the number of flagged positions.
    """
    gm = _f64(global_mask)
    B, S = gm.shape
    idx = np.empty((B, S), np.int32)
    cnt = np.empty(B, np.int32)
    for b in range(B):
        flagged = []
        others = []
        for s in range(S):
            if gm[b, s] == 0.0:
                flagged.append(s)
            else:
                others.append(s)
        idx[b] = np.array(flagged + others[::-1], dtype=np.int32)
        cnt[b] = len(flagged)
    return idx, cnt


# ---------------------------------------------------------------------------
# [FT-LF "Longformer Encoder 计算流程", preprocessing, second item]: the local
# mask becomes an additive score bias through fma(mask, 10000, -10000) in fp32.
# ---------------------------------------------------------------------------
def mask_shift(local_mask, dtype: str) -> torch.Tensor:
    """bias = round_T(round_fp32(10000 * m - 10000)), both roundings to nearest even.

    1 -> 0 and 0 -> -10000 (bf16: -9984, the nearest bf16 value).  The float64
    product and difference are exact for every input whose significand has at
    most 24 bits and whose magnitude keeps 10000*m - 10000 within 53 bits, which
    covers fp16, bf16 and ordinary fp32 masks, so the only roundings are the fp32
    one the page's fma performs and the final store in the activation dtype.
    """
    m = _f64(local_mask)
    exact = m * 10000.0 - 10000.0
    as_f32 = torch.from_numpy(exact).to(torch.float32)
    return as_f32.to(_TORCH[dtype])


def _softmax_weights(scores: np.ndarray) -> np.ndarray:
    e = np.exp(scores - scores.max())
    return e / e.sum()


# ---------------------------------------------------------------------------
# [FT-LF "Longformer Encoder 计算流程", per-layer step 3 and step 4]: local
# sliding-window attention plus global attention, joined by one masked softmax:
# a local token normalises over its window and the global tokens; a global token
# normalises over the whole sequence; padded rows are zeroed.
# ---------------------------------------------------------------------------
class _BatchRow:
    """Per batch row: global positions P (ascending), membership, live positions."""

    def __init__(self, lm_b: np.ndarray, idx_b: np.ndarray, n: int, G: int, b: int):
        if n > G:
            raise ValueError(f"batch row {b} has {n} global tokens, more than G={G}")
        S = lm_b.shape[0]
        self.gpos = idx_b[:n]
        self.is_global = np.zeros(S, bool)
        self.is_global[self.gpos] = True
        self.valid = lm_b == 1.0
        self.S = S


def _row(ctx: _BatchRow, qh, kh, vh, qgh, kgh, vgh, W: int, s: int, scale: float):
    """Output row s of one (b, h) head by the definition (float64 inputs)."""
    if not ctx.valid[s]:                                # R7
        return np.zeros(qh.shape[-1])
    if ctx.is_global[s]:                                # global row: all live keys (R6)
        r = int(np.flatnonzero(ctx.gpos == s)[0])       # R10
        keys = np.flatnonzero(ctx.valid)
        qrow, kk, vv = qgh[r], kgh[keys], vgh[keys]
    else:                                               # local row
        half = W // 2                                   # R1
        lo = max(0, s - half)                           # R2
        hi = min(ctx.S - 1, s + half)
        band = np.arange(lo, hi + 1)
        band = band[~ctx.is_global[band] & ctx.valid[band]]    # R3, R6
        glob = ctx.gpos[ctx.valid[ctx.gpos]]                   # R4, R6
        keys = np.concatenate([glob, band])
        qrow, kk, vv = qh[s], kh[keys], vh[keys]
    p = _softmax_weights(scale * (kk @ qrow))
    return p @ vv


def attention(q, k, v, qg, kg, vg, local_mask, global_mask, W: int, G: int,
              scale: float = 0.125, rows=None):
    """Band + global attention, float64.

    q, k, v, kg, vg: [B,H,S,D]; qg: [B,H,G,D]; masks: [B,S] (see module docs).
    Returns out [B,H,S,D] float64, or, if ``rows`` is a sequence of (b, h, s),
    an array [len(rows), D] holding just those rows.

    Row s of (b, h), with P = the global positions of batch row b (R8, R9) and
    live = positions whose local mask is 1:
      * local mask 0         -> zeros                                        (R7)
      * s in P, s = P[r]     -> softmax over keys j in live of
                                scale*<qg[r], kg[j]>, weights on vg[j]
      * otherwise            -> softmax over keys j in
            {j in P, j live} u {|j-s| <= W/2, 0 <= j < S, j not in P, j live}
                                of scale*<q[s], k[j]>, weights on v[j]
    """
    lm = _f64(local_mask)
    idx, cnt = global_partition(global_mask)
    B, H, S, D = q.shape
    ctxs = {}

    def ctx_of(b):
        if b not in ctxs:
            ctxs[b] = _BatchRow(lm[b], idx[b], int(cnt[b]), G, b)
        return ctxs[b]

    def head(b, h):
        return (_f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]),
                _f64(qg[b, h]), _f64(kg[b, h]), _f64(vg[b, h]))

    if rows is None:
        out = np.zeros((B, H, S, D))
        for b in range(B):
            c = ctx_of(b)
            for h in range(H):
                hd = head(b, h)
                for s in range(S):
                    out[b, h, s] = _row(c, *hd, W, s, scale)
        return out
    out = np.zeros((len(rows), D))
    by_head = {}
    for i, (b, h, s) in enumerate(rows):
        by_head.setdefault((b, h), []).append((i, s))
    for (b, h), items in by_head.items():
        c = ctx_of(b)
        hd = head(b, h)
        for i, s in items:
            out[i] = _row(c, *hd, W, s, scale)
    return out


# ---------------------------------------------------------------------------
# Encoder layer: [FT-LF "Longformer Encoder 计算流程", per-layer steps 1-6].
# ---------------------------------------------------------------------------
def gelu(x):
    """Exact GELU, x * Phi(x), with Phi the standard normal CDF (R11)."""
    x = np.asarray(x, np.float64)
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def layernorm(z, gamma, beta, eps: float = 1e-5):
    """(z - mean) / sqrt(biased var + eps) * gamma + beta over the last axis (R11)."""
    z = np.asarray(z, np.float64)
    mean = z.mean(axis=-1, keepdims=True)
    var = ((z - mean) ** 2).mean(axis=-1, keepdims=True)
    return (z - mean) / np.sqrt(var + eps) * _f64(gamma) + _f64(beta)


def ffn_block(h, resid, w1, b1, w2, b2, ln_g, ln_b, eps: float = 1e-5):
    """Step 6: LN(resid + GELU(h W_1^T + b_1) W_2^T + b_2) over rows of [M, D].

    ``h`` is the FFN input and ``resid`` the residual added after the second
    projection (in the layer both are h1; they are separate here so that a caller
    can hand in the two copies it keeps, e.g. a rounded GEMM input and a wider
    residual).  Weights [out, in]: W_1 [F, D], W_2 [D, F].
    """
    f = gelu(_f64(h) @ _f64(w1).T + _f64(b1))
    return layernorm(_f64(resid) + f @ _f64(w2).T + _f64(b2), ln_g, ln_b, eps)


def layer_projections(x, w, H: int, G: int, global_mask=None):
    """Step 1-2: the five projections of x plus the global query of the global tokens.

    Weights are [out, in] row-major: y = x @ W^T + b.  w_proj stacks the
    Q, K, V, global-K, global-V blocks along its rows; inside each block head h
    owns rows 64h .. 64h+63.  Returns q, k, v, kg, vg [B,H,S,d] and qg [B,H,G,d].

    The global query is projected from the global tokens themselves: qg row r of
    batch row b comes from x[b, p] with p the r-th entry of the global partition
    (R9, R10: the r-th global position for r < n_b; rows from n_b on, which the
    attention never reads, come from the partition's remaining entries).  With the
    global tokens leading this is x[b, r] for every row the attention reads.
    Without ``global_mask`` the first G tokens are taken.
    """
    xd = _f64(x)
    B, S, D = xd.shape
    d = D // H
    proj = xd @ _f64(w["w_proj"]).T + _f64(w["b_proj"])          # [B,S,5D]
    parts = []
    for i in range(5):
        blk = proj[:, :, i * D:(i + 1) * D].reshape(B, S, H, d)
        parts.append(np.ascontiguousarray(blk.transpose(0, 2, 1, 3)))
    if global_mask is None:
        src = xd[:, :G, :]
    else:
        idx, _ = global_partition(global_mask)
        src = np.stack([xd[b, idx[b, :G]] for b in range(B)]) if G > 0 else xd[:, :0, :]
    qg = src @ _f64(w["w_qg"]).T + _f64(w["b_qg"])                 # [B,G,D]
    qg = np.ascontiguousarray(qg.reshape(B, G, H, d).transpose(0, 2, 1, 3))
    q, k, v, kg, vg = parts
    return q, k, v, qg, kg, vg


def encoder_layer(x, w, local_mask, global_mask, H: int, W: int, G: int,
                  scale: float = 0.125, eps: float = 1e-5, rows=None):
    """One Longformer encoder layer, float64, post-LayerNorm order.

      [q|k|v|kg|vg] = x W_proj^T + b_proj;  qg = x[global positions] W_qg^T + b_qg
      a  = band + global attention, heads concatenated      -> [B,S,D]
      h1 = LN(x + a W_o^T + b_o; ln1)
      y  = LN(h1 + GELU(h1 W_1^T + b_1) W_2^T + b_2; ln2)

    ``rows``: optional sequence of (b, s); then only those output rows are
    computed (the projections still cover every token, since attention reads
    them) and an array [len(rows), D] is returned.
    """
    xd = _f64(x)
    B, S, D = xd.shape
    q, k, v, qg, kg, vg = layer_projections(x, w, H, G, global_mask)
    if rows is None:
        a = attention(q, k, v, qg, kg, vg, local_mask, global_mask, W, G, scale)
        a = a.transpose(0, 2, 1, 3).reshape(B, S, D)
        xr = xd
    else:
        rr = [(b, h, s) for (b, s) in rows for h in range(H)]
        a = attention(q, k, v, qg, kg, vg, local_mask, global_mask, W, G, scale, rows=rr)
        a = a.reshape(len(rows), D)
        xr = np.stack([xd[b, s] for (b, s) in rows]) if len(rows) else np.zeros((0, D))
    h1 = layernorm(xr + a @ _f64(w["w_o"]).T + _f64(w["b_o"]), w["ln1_g"], w["ln1_b"], eps)
    return ffn_block(h1, h1, w["w_ffn1"], w["b_ffn1"], w["w_ffn2"], w["b_ffn2"], w["ln2_g"],
                     w["ln2_b"], eps)


# ---------------------------------------------------------------------------
# Algorithmic work (used for throughput accounting, not for parity).
# ---------------------------------------------------------------------------
def allowed_pairs(local_mask, global_mask, W: int, G: int) -> int:
    """Number of allowed (row, key) pairs per head, summed over batch rows.

    Counted by enumerating the definition above; multiply by H for the whole
    problem.  Padded rows contribute nothing.
    """
    lm = _f64(local_mask)
    idx, cnt = global_partition(global_mask)
    B, S = lm.shape
    total = 0
    for b in range(B):
        gpos = idx[b, :cnt[b]]
        is_global = np.zeros(S, bool)
        is_global[gpos] = True
        valid = lm[b] == 1.0
        n_live = int(valid.sum())
        live_glob = int(valid[gpos].sum())
        # prefix count of keys that are live and not global, for band ranges
        ok = (valid & ~is_global).astype(np.int64)
        pref = np.concatenate([[0], np.cumsum(ok)])
        for s in range(S):
            if not valid[s]:
                continue
            if is_global[s]:
                total += n_live
            else:
                lo = max(0, s - W // 2)
                hi = min(S - 1, s + W // 2)
                total += live_glob + int(pref[hi + 1] - pref[lo])
    return total
