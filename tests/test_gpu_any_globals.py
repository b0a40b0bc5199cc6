"""GPU parity of the globals-anywhere attention entry point against the float64 oracle.

The oracle is the plain definition with the global positions taken from the global
mask wherever they are (pinned against a dense brute force with scattered globals in
the oracle tests).  [FT-LF] computation flow, per-layer steps 3-4, without the
head-of-sequence constraint of section "使用前提：四条硬性约束".  Tolerances as for
the leading-globals entry point: fp32 1e-5, fp16 3e-3, bf16 1e-2 max abs error.
With leading global tokens the two entry points must agree bit for bit (same
arithmetic, the index only reorders nothing)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import report

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "fp16": 3e-3, "bf16": 1e-2}


@pytest.fixture(scope="module")
def lf():
    import sparse_long_sequence_amd as m
    m.load_library()
    return m


def _gpu(inp):
    return {n: t.cuda() for n, t in inp.items()}


def _run_any(lf, g, W, G):
    return lf.attn_forward_any_globals(g["q"], g["k"], g["v"], g["qg"], g["kg"], g["vg"],
                                       g["local_mask"], g["global_mask"], W, G)


def _run_lead(lf, g, W, G):
    return lf.attn_forward(g["q"], g["k"], g["v"], g["qg"], g["kg"], g["vg"], g["local_mask"],
                           g["global_mask"], W, G)


def _oracle(inp, W, G, rows=None):
    return oracle.attention(inp["q"], inp["k"], inp["v"], inp["qg"], inp["kg"], inp["vg"],
                            inp["local_mask"], inp["global_mask"], W, G, rows=rows)


def _positions(seed, B, S, n, live_len=None):
    """n distinct sorted positions per batch row, drawn below live_len[b] (default S)."""
    rng = np.random.default_rng(seed)
    out = []
    for b in range(B):
        hi = S if live_len is None else live_len[b]
        out.append(sorted(int(x) for x in rng.choice(hi, n[b] if isinstance(n, list) else n,
                                                     replace=False)))
    return out


def _compare_full(lf, inp, W, G, dtype, case="any"):
    g = _gpu(inp)
    out = _run_any(lf, g, W, G)
    torch.cuda.synchronize()
    got = out.cpu()
    assert torch.isfinite(got.float()).all()
    ref = _oracle(inp, W, G)
    err = report(f"{case} {dtype}", got.double().numpy(), ref, TOL[dtype])
    assert err <= TOL[dtype], f"max abs err {err:.3e} (tol {TOL[dtype]})"
    live = (inp["local_mask"] == 1).numpy()
    o = got.float().numpy()
    for b in range(o.shape[0]):
        pad = o[b][:, ~live[b]]
        assert np.all(pad == 0.0) and not np.any(np.signbit(pad)), "padded rows must be +0.0"
    return got


@pytest.mark.parametrize("dtype", ["fp16", "bf16", "fp32"])
@pytest.mark.parametrize("case", [
    # B, H, S, W, G, pad
    (1, 4, 1024, 256, 8, None),
    (2, 2, 1024, 128, 33, (0.1, 0.25)),
])
def test_leading_globals_match_the_leading_entry_point_bitwise(lf, dtype, case):
    B, H, S, W, G, pad = case
    inp = workloads.random_attention_inputs(40 + G, B, H, S, W, G, dtype, pad_frac=pad)
    g = _gpu(inp)
    a = _run_any(lf, g, W, G)
    b = _run_lead(lf, g, W, G)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16) if dtype != "fp32" else a.view(torch.int32),
                       b.view(torch.int16) if dtype != "fp32" else b.view(torch.int32))


# B, H, S, W, G, positions (per batch row, or ("rand", n) drawn with the case seed), pad
SCATTER_CASES = [
    # tile edges (128 / 256 rows), both sequence ends, adjacent runs, fewer than G
    (2, 2, 1024, 128, 8, [[0, 127, 128, 500, 511, 512, 1000, 1023], [17, 300, 301, 302]], None),
    # more than one 32-row split block and a nearly full 64-key global entry
    (1, 2, 768, 256, 40, ("rand", 40), None),
    # two global-key entries (G > 64)
    (1, 2, 1024, 256, 70, ("rand", 70), None),
    # padding (globals inside the live part), rows beyond the last full tile
    (2, 2, 384, 96, 5, ("live", 5), (0.1, 0.3)),
    # globals only at the end of the sequence
    (1, 2, 512, 64, 4, [[508, 509, 510, 511]], None),
    # capacity but no global token at all
    (1, 2, 512, 64, 6, [[]], None),
]


def _scatter_inputs(ci, dtype):
    B, H, S, W, G, pos, pad = SCATTER_CASES[ci]
    seed = 900 + ci
    if isinstance(pos, tuple):
        if pos[0] == "live":
            # draw the padding first (same draw as the generator), keep globals live
            probe = workloads.random_attention_inputs(seed, B, H, S, W, G, dtype, pad_frac=pad)
            live_len = [int((probe["local_mask"][b] == 1).sum()) for b in range(B)]
            pos = _positions(seed, B, S, pos[1], live_len)
        else:
            pos = _positions(seed, B, S, pos[1])
    inp = workloads.random_attention_inputs(seed, B, H, S, W, G, dtype, pad_frac=pad,
                                            global_positions=pos)
    return inp, W, G


@pytest.mark.parametrize("dtype", ["fp16", "bf16", "fp32"])
@pytest.mark.parametrize("ci", range(len(SCATTER_CASES)))
def test_scattered_globals_full_output(lf, dtype, ci):
    inp, W, G = _scatter_inputs(ci, dtype)
    _compare_full(lf, inp, W, G, dtype, f"scatter {ci}")


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("ci", range(len(SCATTER_CASES)))
def test_scattered_globals_full_output_split_path(lf, dtype, ci, monkeypatch):
    # these grids leave CUs idle, so by default the global rows run in workgroups of
    # their own; LF_ATTN_NO_GWG=1 sends them through the key-split path (gathered
    # global-key entries, split rounds, ticketed combine writing through the index)
    monkeypatch.setenv("LF_ATTN_NO_GWG", "1")
    inp, W, G = _scatter_inputs(ci, dtype)
    _compare_full(lf, inp, W, G, dtype, f"scatter-split {ci}")


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("ci", range(len(SCATTER_CASES)))
def test_scattered_globals_full_output_4wave_layout(lf, dtype, ci, monkeypatch):
    # the 4-wave layout long sequences take (LF_ATTN_WAVES=4), with the key-split path
    monkeypatch.setenv("LF_ATTN_WAVES", "4")
    monkeypatch.setenv("LF_ATTN_NO_GWG", "1")
    inp, W, G = _scatter_inputs(ci, dtype)
    _compare_full(lf, inp, W, G, dtype, f"scatter-4wave {ci}")


@pytest.mark.parametrize("layout", ["4", "8"])
def test_scattered_globals_long_sequence_both_layouts(lf, layout, monkeypatch):
    # 8192 tokens, 16 globals spread over the sequence, 8 heads: 512 workgroups in the
    # 4-wave layout (the second dispatch generation runs its split first), splits of
    # two rounds over gathered global entries
    monkeypatch.setenv("LF_ATTN_WAVES", layout)
    B, H, S, W, G = 1, 8, 8192, 512, 16
    pos = _positions(8192, B, S, G)
    inp = workloads.random_attention_inputs(8192, B, H, S, W, G, "fp16", global_positions=pos)
    _compare_full(lf, inp, W, G, "fp16", f"scatter-long-{layout}wave")


def test_scattered_globals_stress_scale_fp16(lf):
    # N(0,1) inputs: large scores exercise the running max and its rescaling
    B, H, S, W, G = 1, 2, 1024, 256, 16
    pos = _positions(77, B, S, G)
    inp = workloads.random_attention_inputs(77, B, H, S, W, G, "fp16", std=1.0,
                                            global_positions=pos)
    _compare_full(lf, inp, W, G, "fp16", "scatter stress std1")


def test_scattered_globals_longformer_large_shape_every_element(lf):
    # the benchmark shape (B=1 H=16 S=4096 W=512 G=8 fp16) with the 8 global tokens
    # spread over the sequence (tile edges, the middle, both ends): this grid takes the
    # key-split path (gathered entries, 16 splits per head, ticketed combine writing
    # through the index); every output element against the oracle
    B, H, S, W, G = 1, 16, 4096, 512, 8
    pos = [[0, 255, 256, 1000, 2047, 2048, 3500, 4095]]
    inp = workloads.random_attention_inputs(20260102, B, H, S, W, G, "fp16", global_positions=pos)
    g = _gpu(inp)
    out = _run_any(lf, g, W, G)
    out2 = _run_any(lf, g, W, G)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), "not deterministic"
    got = out.cpu()
    assert torch.isfinite(got.float()).all()
    ref = _oracle(inp, W, G)
    err = report("scatter longformer-large fp16", got.double().numpy(), ref, TOL["fp16"])
    assert err <= TOL["fp16"], f"max abs err {err:.3e}"


# ------------------------------------------------------------------ encoder layer / stack
# [FT-LF] computation flow, per-layer steps 1-6, with the global tokens anywhere: the
# global queries come from the global tokens (oracle reading R10, pinned against the
# torch-composed dense layer), the attention is the globals-anywhere attention.
# Tolerances as for the leading-globals layer: fp16 3e-3, bf16 2.5e-2 + 2^-8 |ref|,
# fp32 1e-4 (derivations in tests/test_gpu_layer.py).
LAYER_TOL = {"fp16": 3e-3, "bf16": 2.5e-2, "fp32": 1e-4}


def _layer_inputs(seed, B, S, D, F, G, dtype, positions=None, pad=None):
    rng = np.random.default_rng(seed)
    w = workloads.random_layer_params(rng, D, F, dtype, w_std=0.05, b_std=0.02, ln_jitter=0.1)
    x = torch.from_numpy(rng.standard_normal((B, S, D))).to(workloads.TORCH_DTYPES[dtype])
    lm, gm = workloads.make_masks(rng, B, S, G, dtype, pad, None, positions)
    return x, w, lm, gm


def _bits(t):
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16)


@pytest.mark.parametrize("dtype", ["fp16", "bf16", "fp32"])
def test_layer_any_equals_layer_with_leading_globals(lf, dtype):
    B, S, D, H, F, W, G = 2, 512, 256, 4, 512, 128, 8
    x, w, lm, gm = _layer_inputs(61, B, S, D, F, G, dtype, pad=(0.1, 0.2))
    xg, lmg, gmg = x.cuda(), lm.cuda(), gm.cuda()
    wg = {n: t.cuda() for n, t in w.items()}
    a = lf.encoder_layer(xg, wg, lmg, gmg, H, W, G, any_globals=True)
    b = lf.encoder_layer(xg, wg, lmg, gmg, H, W, G)
    torch.cuda.synchronize()
    if dtype == "fp32":
        # the vector-ALU kernel starts its band chunks at another key: sums reorder
        assert (a - b).abs().max().item() <= 1e-6
    else:
        assert torch.equal(_bits(a), _bits(b))


@pytest.mark.parametrize("dtype", ["fp16", "bf16", "fp32"])
@pytest.mark.parametrize("case", [
    # B, S, D, H, F, W, G, positions, pad
    (2, 512, 256, 4, 512, 128, 8, [[3, 100, 101, 255, 256, 400, 500, 511], [0, 64, 300]], None),
    (1, 384, 512, 8, 1024, 64, 5, [[10, 200, 201, 300, 301]], (0.1, 0.15)),
], ids=["B2_S512_G8", "B1_S384_G5_pad"])
@pytest.mark.parametrize("split_path", [False, True], ids=["default", "split_path"])
def test_layer_any_scattered_globals_vs_oracle(lf, dtype, case, split_path, monkeypatch):
    if split_path:
        if dtype == "fp32":
            pytest.skip("fp32 attention has one global-row path, split over keys whenever the "
                        "sequence spans more than one 256-row tile; the default case runs it")
        monkeypatch.setenv("LF_ATTN_NO_GWG", "1")
    B, S, D, H, F, W, G, positions, pad = case
    x, w, lm, gm = _layer_inputs(71 + S, B, S, D, F, G, dtype, positions, pad)
    live = lm.float()
    for b in range(B):
        assert all(live[b, p] == 1 for p in positions[b]), "keep the globals unpadded"
    y = lf.encoder_layer(x.cuda(), {n: t.cuda() for n, t in w.items()}, lm.cuda(), gm.cuda(),
                         H, W, G, any_globals=True)
    torch.cuda.synchronize()
    got = y.cpu()
    assert torch.isfinite(got.float()).all()
    ref = oracle.encoder_layer(x, w, lm, gm, H, W, G)
    err = np.abs(got.double().numpy() - ref)
    tol = LAYER_TOL[dtype] + (2.0 ** -8 * np.abs(ref) if dtype == "bf16" else 0.0)
    report(f"layer-any S{S} G{G} {dtype}{' split' if split_path else ''}", got.double().numpy(),
           ref, LAYER_TOL[dtype] if dtype != "bf16" else "per-element")
    assert np.all(err <= tol), f"max abs err {err.max():.3e}"


@pytest.mark.parametrize("dtype", ["fp16", "fp32"])
def test_stack_any_equals_layer_any_after_layer_any(lf, dtype):
    B, S, D, H, F, W, G, L = 1, 512, 256, 4, 512, 128, 6, 3
    rng = np.random.default_rng(81)
    layers = [workloads.random_layer_params(rng, D, F, dtype, w_std=0.05, b_std=0.02,
                                            ln_jitter=0.1) for _ in range(L)]
    x = torch.from_numpy(rng.standard_normal((B, S, D))).to(workloads.TORCH_DTYPES[dtype])
    lm, gm = workloads.make_masks(rng, B, S, G, dtype, None, None, [[7, 130, 131, 260, 390, 505]])
    xg, lmg, gmg = x.cuda(), lm.cuda(), gm.cuda()
    wg = [{n: t.cuda() for n, t in w.items()} for w in layers]
    y = lf.encoder_forward(xg, wg, lmg, gmg, H, W, G, any_globals=True)
    cur = xg
    for w in wg:
        cur = lf.encoder_layer(cur, w, lmg, gmg, H, W, G, any_globals=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y), _bits(cur))


def test_layer_any_full_size_every_element(lf):
    # the graded layer shape (B=2 S=4096 hidden 1024, 16 heads, FFN 4096, W=512) with its
    # 16 global tokens spread over each sequence; every output element
    wl = workloads.LAYER_FP16
    t = workloads.make_layer_inputs(wl)
    rng = np.random.default_rng(wl.seed + 11)
    positions = [sorted(int(p) for p in rng.choice(wl.S, wl.G, replace=False)) for _ in range(wl.B)]
    gm = torch.full((wl.B, wl.S), workloads.NOT_GLOBAL).to(workloads.TORCH_DTYPES[wl.dtype])
    for b in range(wl.B):
        gm[b, positions[b]] = 0.0
    x, lm = t["x"], t["local_mask"]
    w = {n: t[n] for n in lf.LAYER_WEIGHT_FIELDS}
    y = lf.encoder_layer(x.cuda(), {n: v.cuda() for n, v in w.items()}, lm.cuda(), gm.cuda(),
                         wl.H, wl.W, wl.G, any_globals=True)
    torch.cuda.synchronize()
    got = y.cpu()
    assert torch.isfinite(got.float()).all()
    ref = oracle.encoder_layer(x, w, lm, gm, wl.H, wl.W, wl.G)
    err = report("layer-any full size fp16", got.double().numpy(), ref, LAYER_TOL["fp16"])
    assert err <= LAYER_TOL["fp16"], f"max abs err {err:.3e}"


def test_stack_any_last_layer_matches_oracle(lf):
    # two layers with the global tokens scattered: the stack's output against the
    # oracle layer applied to the GPU's first-layer output
    B, S, D, H, F, W, G = 1, 512, 256, 4, 512, 128, 6
    rng = np.random.default_rng(91)
    layers = [workloads.random_layer_params(rng, D, F, "fp16", w_std=0.05, b_std=0.02,
                                            ln_jitter=0.1) for _ in range(2)]
    x = torch.from_numpy(rng.standard_normal((B, S, D))).to(torch.float16)
    lm, gm = workloads.make_masks(rng, B, S, G, "fp16", None, None, [[3, 130, 131, 260, 390, 500]])
    xg, lmg, gmg = x.cuda(), lm.cuda(), gm.cuda()
    wg = [{n: t.cuda() for n, t in w.items()} for w in layers]
    y1 = lf.encoder_layer(xg, wg[0], lmg, gmg, H, W, G, any_globals=True)
    y = lf.encoder_forward(xg, wg, lmg, gmg, H, W, G, any_globals=True)
    torch.cuda.synchronize()
    ref = oracle.encoder_layer(y1.cpu(), layers[1], lm, gm, H, W, G)
    err = report("stack-any last layer fp16", y.cpu().double().numpy(), ref, LAYER_TOL["fp16"])
    assert err <= LAYER_TOL["fp16"], f"max abs err {err:.3e}"
