"""Pins for the float64 oracle: each check fixes the oracle to something other than itself.

* hand-derived fixtures under tests/golden/ (partition, mask shift, a worked
  attention example, explicit band supports);
* a dense boolean-mask formulation through torch library routines
  (tests/dense_reference.py) on random small inputs, including padding,
  G = 0 and global tokens away from the head of the sequence;
* closed forms and invariants: rows sum to 1, q = 0 gives the mean of the
  allowed v rows, global rows equal full masked attention, a wide window with
  no globals is full attention, padded rows are exactly +0.0;
* textbook GELU values and LayerNorm moments; the layer against torch's
  linear / layer_norm / gelu composition.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
from tests.dense_reference import dense_attention, dense_layer
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------- partition
def test_partition_golden():
    for case in _load("partition_small.json")["cases"]:
        idx, cnt = oracle.global_partition(np.array(case["global_mask"]))
        assert idx.tolist() == case["global_idx"]
        assert cnt.tolist() == case["global_count"]


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 3), st.integers(1, 70), st.data())
def test_partition_invariants(B, S, data):
    flags = np.array(data.draw(st.lists(st.booleans(), min_size=B * S, max_size=B * S)))
    gm = np.where(flags.reshape(B, S), 0.0, -10000.0)
    idx, cnt = oracle.global_partition(gm)
    for b in range(B):
        n = cnt[b]
        assert n == flags.reshape(B, S)[b].sum()
        assert sorted(idx[b].tolist()) == list(range(S))         # a permutation
        head, tail = idx[b, :n], idx[b, n:]
        assert np.all(gm[b, head] == 0.0) and np.all(np.diff(head) > 0)
        assert np.all(gm[b, tail] != 0.0) and np.all(np.diff(tail) < 0)


# --------------------------------------------------------------------------- mask shift
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_mask_shift_golden(dtype):
    cases = _load("mask_shift_values.json")["cases"][dtype]
    m = torch.tensor([[c[0] for c in cases]], dtype=workloads.TORCH_DTYPES[dtype])
    got = oracle.mask_shift(m, dtype)
    assert got.dtype == workloads.TORCH_DTYPES[dtype]
    assert got.to(torch.float64).tolist()[0] == [c[1] for c in cases]


# --------------------------------------------------------------------------- attention
def test_attention_worked_example():
    ex = _load("attention_worked_example.json")
    inp = ex["inputs"]
    t = {n: np.array(inp[n], np.float64).reshape(1, 1, -1, 1) for n in
         ("q", "k", "v", "qg", "kg", "vg")}
    gm = np.array([inp["global_mask"]])
    for case in ex["cases"]:
        lm = np.array([case["local_mask"]])
        out = oracle.attention(t["q"], t["k"], t["v"], t["qg"], t["kg"], t["vg"], lm, gm,
                               W=2, G=1)
        np.testing.assert_allclose(out.reshape(-1), case["out"], rtol=0, atol=1e-15)


def test_band_support_identity_values():
    ex = _load("band_support_S64_W16_G2.json")
    S, W, G = 64, 16, 2
    z = np.zeros((1, 1, S, 64))
    eye = np.eye(64).reshape(1, 1, S, 64)
    lm = np.ones((1, S))
    gm = np.full((1, S), -10000.0)
    gm[0, :G] = 0.0
    out = oracle.attention(z, z, eye, np.zeros((1, 1, G, 64)), z, eye, lm, gm, W, G)
    for row, ranges in ex["rows"].items():
        keys = [j for lo, hi in ranges for j in range(lo, hi + 1)]
        expect = np.zeros(64)
        expect[keys] = 1.0 / len(keys)
        np.testing.assert_allclose(out[0, 0, int(row)], expect, rtol=0, atol=1e-15)


def _random_problem(seed, B, H, S, W, G, n_glob, pad, lead, D=8, std=1.0):
    rng = np.random.default_rng(seed)
    t = {n: rng.standard_normal((B, H, S if n != "qg" else G, D)) * std
         for n in ("q", "k", "v", "qg", "kg", "vg")}
    lm = np.ones((B, S))
    gm = np.full((B, S), -10000.0)
    for b in range(B):
        pos = np.arange(n_glob) if lead else np.sort(rng.choice(S, n_glob, replace=False))
        gm[b, pos] = 0.0
        if pad:
            npad = int(rng.integers(0, S // 2 + 1))
            if npad:
                lm[b, S - npad:] = 0.0
            if not lead and npad:
                # padding in the middle too: knock out a few random positions
                lm[b, rng.choice(S, min(3, S), replace=False)] = 0.0
    return t, lm, gm


@settings(max_examples=40, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), B=st.integers(1, 2), H=st.integers(1, 2),
       S=st.integers(2, 80), halfw=st.integers(1, 40), gfrac=st.floats(0, 0.5),
       pad=st.booleans(), lead=st.booleans())
def test_attention_matches_dense_bruteforce(seed, B, H, S, halfw, gfrac, pad, lead):
    W = 2 * halfw
    n_glob = int(gfrac * S)
    G = n_glob + 1
    t, lm, gm = _random_problem(seed, B, H, S, W, G, n_glob, pad, lead)
    got = oracle.attention(t["q"], t["k"], t["v"], t["qg"], t["kg"], t["vg"], lm, gm, W, G)
    ref = dense_attention(t["q"], t["k"], t["v"], t["qg"], t["kg"], t["vg"], lm, gm, W)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_rows_sum_to_one_and_padded_rows_are_plus_zero():
    B, H, S, W, G = 2, 2, 96, 16, 5
    t, lm, gm = _random_problem(7, B, H, S, W, G, 5, pad=True, lead=True, std=2.0)
    ones = np.ones_like(t["v"])
    out = oracle.attention(t["q"], t["k"], ones, t["qg"], t["kg"], ones, lm, gm, W, G)
    live = lm == 1
    for b in range(B):
        np.testing.assert_allclose(out[b][:, live[b]], 1.0, rtol=0, atol=1e-14)
        pad_rows = out[b][:, ~live[b]]
        assert np.all(pad_rows == 0.0) and not np.any(np.signbit(pad_rows))


def test_zero_query_is_mean_of_allowed_values():
    # q = qg = 0: every allowed key has the same weight (closed form)
    B, H, S, W, G = 1, 1, 40, 8, 3
    t, lm, gm = _random_problem(11, B, H, S, W, G, 3, pad=False, lead=True)
    z = np.zeros_like(t["q"])
    zg = np.zeros_like(t["qg"])
    out = oracle.attention(z, t["k"], t["v"], zg, t["kg"], t["vg"], lm, gm, W, G)
    v, vg = t["v"][0, 0], t["vg"][0, 0]
    for s in range(S):
        if s < G:
            expect = vg.mean(axis=0)
        else:
            keys = sorted(set(range(G)) | set(range(max(G, s - 4), min(S, s + 5))))
            expect = v[keys].mean(axis=0)
        np.testing.assert_allclose(out[0, 0, s], expect, rtol=0, atol=1e-14)


def test_global_rows_equal_full_attention():
    B, H, S, W, G = 1, 2, 64, 8, 4
    t, lm, gm = _random_problem(3, B, H, S, W, G, 4, pad=False, lead=True, std=1.5)
    out = oracle.attention(t["q"], t["k"], t["v"], t["qg"], t["kg"], t["vg"], lm, gm, W, G)
    full = F.scaled_dot_product_attention(torch.tensor(t["qg"]), torch.tensor(t["kg"]),
                                          torch.tensor(t["vg"]), scale=0.125).numpy()
    np.testing.assert_allclose(out[:, :, :G], full, rtol=1e-12, atol=1e-14)


def test_wide_window_without_globals_is_full_attention():
    # W >= 2(S-1) and no global token: every row sees every key
    B, H, S = 1, 2, 33
    W = 2 * S
    t, lm, gm = _random_problem(5, B, H, S, W, 1, 0, pad=False, lead=True, std=1.5)
    out = oracle.attention(t["q"], t["k"], t["v"], t["qg"], t["kg"], t["vg"], lm, gm, W, 1)
    full = F.scaled_dot_product_attention(torch.tensor(t["q"]), torch.tensor(t["k"]),
                                          torch.tensor(t["v"]), scale=0.125).numpy()
    np.testing.assert_allclose(out, full, rtol=1e-12, atol=1e-14)


def test_no_globals_is_sliding_window():
    B, H, S, W = 1, 1, 50, 10
    t, lm, gm = _random_problem(9, B, H, S, W, 0, 0, pad=False, lead=True)
    out = oracle.attention(t["q"], t["k"], t["v"], t["qg"][:, :, :0], t["kg"], t["vg"],
                           lm, gm, W, 0)
    q, k, v = t["q"][0, 0], t["k"][0, 0], t["v"][0, 0]
    for s in (0, 3, 25, 49):
        keys = np.arange(max(0, s - 5), min(S, s + 6))
        e = 0.125 * k[keys] @ q[s]
        p = torch.softmax(torch.tensor(e), 0).numpy()
        np.testing.assert_allclose(out[0, 0, s], p @ v[keys], rtol=1e-12, atol=1e-14)


def test_too_many_globals_raises():
    gm = np.zeros((1, 8))
    lm = np.ones((1, 8))
    z = np.zeros((1, 1, 8, 4))
    with pytest.raises(ValueError):
        oracle.attention(z, z, z, z[:, :, :2], z, z, lm, gm, 4, 2)


def test_rows_subset_matches_full():
    B, H, S, W, G = 2, 2, 48, 12, 3
    t, lm, gm = _random_problem(13, B, H, S, W, G, 3, pad=True, lead=True)
    full = oracle.attention(t["q"], t["k"], t["v"], t["qg"], t["kg"], t["vg"], lm, gm, W, G)
    rows = [(0, 1, 0), (1, 0, 47), (1, 1, 20), (0, 0, 2)]
    sub = oracle.attention(t["q"], t["k"], t["v"], t["qg"], t["kg"], t["vg"], lm, gm, W, G,
                           rows=rows)
    for i, (b, h, s) in enumerate(rows):
        assert np.array_equal(sub[i], full[b, h, s])


def test_allowed_pairs_closed_form():
    # unpadded, leading globals: G*S + (S-G)(W+1+G) - (W/2)(W/2+1) per head
    for (S, W, G) in ((64, 16, 2), (4096, 512, 8), (256, 32, 0)):
        lm = np.ones((1, S))
        gm = np.full((1, S), -10000.0)
        gm[0, :G] = 0.0
        expect = G * S + (S - G) * (W + 1 + G) - (W // 2) * (W // 2 + 1)
        assert oracle.allowed_pairs(lm, gm, W, G) == expect


def test_allowed_pairs_matches_dense_count():
    t, lm, gm = _random_problem(17, 2, 1, 70, 12, 6, 5, pad=True, lead=True)
    from tests.dense_reference import dense_masks
    local, glob, is_glob, live = dense_masks(lm, gm, 12)
    rows_glob = (is_glob & live).unsqueeze(-1)
    rows_loc = (~is_glob & live).unsqueeze(-1)
    expect = int((glob & rows_glob).sum() + (local & rows_loc).sum())
    assert oracle.allowed_pairs(lm, gm, 12, 6) == expect


# --------------------------------------------------------------------------- layer parts
def test_gelu_textbook_values():
    # x * Phi(x) with Phi(1) = 0.8413447460685429, Phi(2) = 0.9772498680518208
    np.testing.assert_allclose(oracle.gelu([0.0, 1.0, -1.0, 2.0]),
                               [0.0, 0.8413447460685429, -0.15865525393145707,
                                1.9544997361036416], rtol=0, atol=1e-15)


def test_layernorm_moments_and_small_case():
    z = np.array([[1.0, 2.0, 3.0, 4.0]])
    got = oracle.layernorm(z, np.ones(4), np.zeros(4), eps=1e-5)
    expect = (z - 2.5) / math.sqrt(1.25 + 1e-5)
    np.testing.assert_allclose(got, expect, rtol=0, atol=1e-15)
    rng = np.random.default_rng(1)
    z = rng.standard_normal((5, 64)) * 3 + 1
    y = oracle.layernorm(z, np.ones(64), np.zeros(64), eps=1e-5)
    var = z.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-13)
    np.testing.assert_allclose(y.var(axis=1), var / (var + 1e-5), rtol=1e-12)


def _tiny_layer(seed, B=2, S=48, D=32, H=4, F=64, W=8, G=3, b_std=0.1, ln_jitter=0.1):
    rng = np.random.default_rng(seed)
    w = workloads.random_layer_params(rng, D, F, "fp32", w_std=0.2, b_std=b_std,
                                      ln_jitter=ln_jitter)
    x = torch.tensor(rng.standard_normal((B, S, D)), dtype=torch.float32)
    lm = torch.ones(B, S)
    lm[1, S - 5:] = 0
    gm = torch.full((B, S), -10000.0)
    gm[:, :G] = 0
    return x, w, lm, gm, H, W, G


def test_layer_matches_torch_library_composition():
    x, w, lm, gm, H, W, G = _tiny_layer(21)
    got = oracle.encoder_layer(x, w, lm, gm, H, W, G)
    ref = dense_layer(x, w, lm, gm, H, W, G)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)


def test_layer_with_scattered_globals_matches_torch_library_composition():
    # the global queries come from the global tokens wherever they sit (the dense
    # reference gathers them with torch.nonzero, independently of the oracle's partition)
    x, w, lm, gm, H, W, G = _tiny_layer(24)
    gm = torch.full(gm.shape, -10000.0)
    gm[0, [2, 17, 40]] = 0
    gm[1, [0, 5]] = 0
    got = oracle.encoder_layer(x, w, lm, gm, H, W, G)
    ref = dense_layer(x, w, lm, gm, H, W, G)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)


def test_layer_rows_subset_matches_full():
    x, w, lm, gm, H, W, G = _tiny_layer(22)
    full = oracle.encoder_layer(x, w, lm, gm, H, W, G)
    rows = [(0, 0), (1, 47), (1, 10), (0, 2)]
    sub = oracle.encoder_layer(x, w, lm, gm, H, W, G, rows=rows)
    for i, (b, s) in enumerate(rows):
        np.testing.assert_allclose(sub[i], full[b, s], rtol=0, atol=1e-13)


def test_layer_zero_output_projection_is_layernorm_of_input():
    x, w, lm, gm, H, W, G = _tiny_layer(23, b_std=0.0, ln_jitter=0.0)
    for n in ("w_o", "w_ffn1", "w_ffn2"):
        w[n] = torch.zeros_like(w[n])
    got = oracle.encoder_layer(x, w, lm, gm, H, W, G)
    ln = F.layer_norm(x.double(), (x.shape[-1],), eps=1e-5)
    ln2 = F.layer_norm(ln, (x.shape[-1],), eps=1e-5)   # h1 + GELU(0) W2 = h1
    np.testing.assert_allclose(got, ln2.numpy(), rtol=0, atol=1e-12)


def test_ffn_block_one_hot_closed_form():
    # [FT-LF] per-layer step 6.  A one-hot W1 picks input column 1 into F column 2; a
    # one-hot W2 puts 2x its GELU into output column 3.  A transposed weight, a dropped
    # or misplaced bias, or adding h instead of the residual changes that value (GELU
    # and LayerNorm themselves are pinned above).
    M, D, F = 3, 4, 3
    h = np.array([[0.3, -1.2, 0.7, 2.0], [1.5, 0.4, -0.6, 0.1], [-0.8, 2.2, 0.0, -1.1]])
    resid = np.arange(M * D, dtype=np.float64).reshape(M, D) * 0.25 - 1.0
    w1 = np.zeros((F, D)); w1[2, 1] = 1.0
    b1 = np.array([0.0, 0.0, 0.5])
    w2 = np.zeros((D, F)); w2[3, 2] = 2.0
    b2 = np.array([0.1, 0.2, 0.3, 0.4])
    gamma, beta = np.array([1.0, 2.0, 0.5, 1.0]), np.array([0.0, 0.1, 0.0, -0.2])
    got = oracle.ffn_block(h, resid, w1, b1, w2, b2, gamma, beta)
    for m in range(M):
        z = resid[m] + b2
        z[3] += 2.0 * float(oracle.gelu(h[m, 1] + 0.5))
        mu = z.mean()
        var = ((z - mu) ** 2).mean()
        expect = (z - mu) / math.sqrt(var + 1e-5) * gamma + beta
        np.testing.assert_allclose(got[m], expect, rtol=0, atol=1e-14)


def test_ffn_block_is_the_layer_step():
    # the layer's last step is the FFN block with h = resid = h1: zero attention output
    # projection makes h1 = LN(x), so the layer is ffn_block(LN(x), LN(x), ...)
    x, w, lm, gm, H, W, G = _tiny_layer(25, b_std=0.0, ln_jitter=0.0)
    w["w_o"] = torch.zeros_like(w["w_o"])
    got = oracle.encoder_layer(x, w, lm, gm, H, W, G)
    h1 = F.layer_norm(x.double(), (x.shape[-1],), eps=1e-5).numpy()
    ref = oracle.ffn_block(h1, h1, w["w_ffn1"], w["b_ffn1"], w["w_ffn2"], w["b_ffn2"],
                           w["ln2_g"], w["ln2_b"])
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
