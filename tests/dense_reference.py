"""Dense boolean-mask formulation of band + global attention, for pinning the oracle.

Built from library routines only (torch's scaled_dot_product_attention, linear,
layer_norm, gelu) and an explicit S x S boolean mask written from the rules of
the FasterTransformer Longformer page, section "Longformer Encoder 计算流程",
per-layer steps 3-4.  It is a second, independent formulation: the oracle
enumerates each row's allowed key set, this module masks a full score matrix.
Only small shapes are meant (S up to a few hundred).
"""
import numpy as np
import torch
import torch.nn.functional as F


def _t64(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64)
    return torch.as_tensor(np.asarray(x, np.float64))


def dense_masks(local_mask, global_mask, W):
    """Boolean [B,S,S] masks for local rows and for global rows, plus per-row flags."""
    lm = _t64(local_mask)
    gm = _t64(global_mask)
    B, S = lm.shape
    i = torch.arange(S).view(S, 1)
    j = torch.arange(S).view(1, S)
    in_band = (i - j).abs() <= W // 2                 # [S,S]
    is_glob = gm == 0                                 # [B,S]
    live = lm == 1                                    # [B,S]
    key_glob = is_glob.view(B, 1, S)
    key_live = live.view(B, 1, S)
    local = ((in_band.view(1, S, S) & ~key_glob) | key_glob) & key_live
    glob = key_live.expand(B, S, S)
    return local, glob, is_glob, live


def dense_attention(q, k, v, qg, kg, vg, local_mask, global_mask, W, scale=0.125):
    """out [B,H,S,D] float64 via two masked SDPA calls and a per-row select."""
    q, k, v, qg, kg, vg = (_t64(t) for t in (q, k, v, qg, kg, vg))
    B, H, S, D = q.shape
    local, glob, is_glob, live = dense_masks(local_mask, global_mask, W)
    out_local = F.scaled_dot_product_attention(q, k, v, attn_mask=local.view(B, 1, S, S),
                                               scale=scale)
    # global query for position s: qg row = number of global positions before s
    rank = torch.cumsum(is_glob.to(torch.int64), dim=1) - 1          # [B,S]
    rank = rank.clamp(min=0, max=max(qg.shape[2] - 1, 0))
    if qg.shape[2] > 0:
        qsel = torch.stack([qg[b][:, rank[b]] for b in range(B)])    # [B,H,S,D]
    else:
        qsel = torch.zeros_like(q)
    out_glob = F.scaled_dot_product_attention(qsel, kg, vg, attn_mask=glob.view(B, 1, S, S),
                                              scale=scale)
    sel = is_glob.view(B, 1, S, 1)
    out = torch.where(sel, out_glob, out_local)
    out = torch.where(live.view(B, 1, S, 1), out, torch.zeros(()))
    # rows whose mask row is empty are all-NaN in SDPA; they are padded rows, zeroed above
    return out.numpy()


def dense_layer(x, w, local_mask, global_mask, H, W, G, scale=0.125, eps=1e-5):
    """Encoder layer from torch library routines (linear, layer_norm, gelu) + dense attention."""
    x = _t64(x)
    B, S, D = x.shape
    d = D // H
    ww = {n: _t64(t) for n, t in w.items()}
    proj = F.linear(x, ww["w_proj"], ww["b_proj"])                   # [B,S,5D]

    def heads(t):
        return t.reshape(B, t.shape[1], H, d).transpose(1, 2)

    q, k, v, kg, vg = (heads(proj[..., i * D:(i + 1) * D]) for i in range(5))
    # global queries from the global tokens: row r <- the r-th position whose global-mask
    # value is 0 (rows past the count are never read by the attention: zeros)
    gpos = [torch.nonzero(torch.as_tensor(global_mask)[b] == 0).flatten() for b in range(B)]
    xg = torch.zeros(B, G, D, dtype=x.dtype)
    for b in range(B):
        n = min(G, len(gpos[b]))
        xg[b, :n] = x[b, gpos[b][:n]]
    qg = heads(F.linear(xg, ww["w_qg"], ww["b_qg"]))
    a = torch.as_tensor(dense_attention(q, k, v, qg, kg, vg, local_mask, global_mask, W, scale))
    a = a.transpose(1, 2).reshape(B, S, D)
    h1 = F.layer_norm(x + F.linear(a, ww["w_o"], ww["b_o"]), (D,), ww["ln1_g"], ww["ln1_b"], eps)
    f = F.gelu(F.linear(h1, ww["w_ffn1"], ww["b_ffn1"]))
    y = F.layer_norm(h1 + F.linear(f, ww["w_ffn2"], ww["b_ffn2"]), (D,), ww["ln2_g"], ww["ln2_b"],
                     eps)
    return y.numpy()
