"""GPU parity of band + global attention against the float64 oracle.

[FT-LF] computation flow, per-layer steps 3-4.  Tolerances (max abs error on the
outputs): fp32 1e-5, fp16 3e-3, bf16 1e-2.  Every problem, the full-size
workloads included (in the launch configuration the benchmark times), is compared
element by element over the whole output, plus properties that hold at any size
(padded rows exactly +0.0, finite outputs, determinism).  Each comparison prints
its max abs error and max abs error / max |ref| (tests/parity.py)."""
import zlib

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


def _run(lf, g, W, G, out=None):
    return lf.attn_forward(g["q"], g["k"], g["v"], g["qg"], g["kg"], g["vg"], g["local_mask"],
                           g["global_mask"], W, G, out=out)


def _oracle(inp, W, G, rows=None):
    return oracle.attention(inp["q"], inp["k"], inp["v"], inp["qg"], inp["kg"], inp["vg"],
                            inp["local_mask"], inp["global_mask"], W, G, rows=rows)


def _check_padded_zero(out_cpu, lm):
    live = (lm == 1).numpy()
    o = out_cpu.float().numpy()
    B = o.shape[0]
    for b in range(B):
        pad = o[b][:, ~live[b]]
        assert np.all(pad == 0.0) and not np.any(np.signbit(pad)), "padded rows must be +0.0"


def _full_compare(lf, inp, W, G, dtype, case="attn"):
    g = _gpu(inp)
    out = _run(lf, g, W, G)
    torch.cuda.synchronize()
    got = out.cpu()
    ref = _oracle(inp, W, G)
    assert np.isfinite(got.float().numpy()).all()
    err = report(f"{case} {dtype}", got.double().numpy(), ref, TOL[dtype])
    assert err <= TOL[dtype], f"max abs err {err:.3e} (tol {TOL[dtype]})"
    _check_padded_zero(got, inp["local_mask"])
    return got, ref


# ---------------------------------------------------------------- tiny workload (fp32)
def test_tiny_fp32_workload(lf):
    wl = workloads.TINY_FP32
    inp = workloads.make_attention_inputs(wl)
    _full_compare(lf, inp, wl.W, wl.G, "fp32", wl.name)


# ---------------------------------------------------------------- mid-size, every element
CASES = [
    # B, H, S, W, G, pad, n_global (None = G)
    (1, 2, 64, 16, 2, None, None),       # tiny shape (single ragged tile)
    (2, 3, 1024, 128, 5, (0.1, 0.25), None),
    (1, 2, 384, 96, 7, (0.1, 0.3), None),   # S not a multiple of the 128-row tile
    (1, 2, 1024, 512, 64, None, None),      # a full 64-key global chunk, two 32-row q-blocks
    (2, 2, 1024, 512, 33, (0.05, 0.1), None),
    (1, 2, 768, 256, 0, None, None),         # no global tokens at all
    (1, 1, 256, 2, 1, None, None),           # narrowest window
    (1, 1, 512, 256, 256, None, None),       # G == W: many global rows
    (2, 1, 512, 128, 16, None, (3, 0)),      # fewer globals than capacity, one row none
    (1, 2, 2048, 512, 8, (0.6, 0.7), None),  # heavy padding
    # windows that give the helper-wave layout 4 and 7 band steps (the global keys
    # folded into the first and last of them; the last step alone or second of a pair)
    (2, 2, 1280, 160, 3, (0.1, 0.25), None),
    (1, 3, 1152, 192, 32, None, None),       # G = 32 (every slot of the folded block), ragged tile
    (1, 2, 1536, 384, 17, (0.05, 0.1), None),
]


@pytest.mark.parametrize("dtype", ["fp16", "bf16", "fp32"])
@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}S{c[2]}W{c[3]}G{c[4]}" for c in CASES])
def test_attention_parity_mid(lf, dtype, case):
    B, H, S, W, G, pad, ng = case
    inp = workloads.random_attention_inputs(zlib.crc32(repr(case).encode()) % 100000, B, H, S, W, G, dtype,
                                            pad_frac=pad, n_global=ng)
    _full_compare(lf, inp, W, G, dtype, f"mid B{B}H{H}S{S}W{W}G{G}")


@pytest.mark.parametrize("helpers", ["on", "off"])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}S{c[2]}W{c[3]}G{c[4]}" for c in CASES])
def test_attention_parity_mid_split_path(lf, dtype, case, helpers, monkeypatch):
    # these grids leave CUs idle, so by default the global rows run in workgroups of
    # their own; LF_ATTN_NO_GWG=1 sends them through the key-split path instead, where
    # helper waves compute each tile's split (G <= 32, W >= 160: at least 4 band steps)
    # unless LF_ATTN_NO_HELP=1
    # leaves it to the band waves
    monkeypatch.setenv("LF_ATTN_NO_GWG", "1")
    if helpers == "off":
        monkeypatch.setenv("LF_ATTN_NO_HELP", "1")
    B, H, S, W, G, pad, ng = case
    inp = workloads.random_attention_inputs(zlib.crc32(repr(case).encode()) % 100000, B, H, S, W, G, dtype,
                                            pad_frac=pad, n_global=ng)
    _full_compare(lf, inp, W, G, dtype, f"mid-split B{B}H{H}S{S}W{W}G{G}")


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}S{c[2]}W{c[3]}G{c[4]}" for c in CASES])
def test_attention_parity_mid_4wave_layout(lf, dtype, case, monkeypatch):
    # the 4-wave layout (128-row workgroups, 4-slot ring, a barrier per step) that long
    # sequences take, forced on these shapes (LF_ATTN_WAVES=4, with the key-split path)
    monkeypatch.setenv("LF_ATTN_WAVES", "4")
    monkeypatch.setenv("LF_ATTN_NO_GWG", "1")
    B, H, S, W, G, pad, ng = case
    inp = workloads.random_attention_inputs(zlib.crc32(repr(case).encode()) % 100000, B, H, S, W, G, dtype,
                                            pad_frac=pad, n_global=ng)
    _full_compare(lf, inp, W, G, dtype, f"mid-4wave B{B}H{H}S{S}W{W}G{G}")


LONG_CASES = [
    # B, H, S, W, G, pad: 512 workgroups in the 4-wave layout (two dispatch
    # generations: the second runs its split first), splits of 2 rounds, 2 query blocks
    (1, 8, 8192, 256, 40, None),
    (1, 8, 8192, 512, 8, (0.05, 0.15)),
]


@pytest.mark.parametrize("layout", ["4", "8"])
@pytest.mark.parametrize("case", LONG_CASES, ids=[f"B{c[0]}H{c[1]}S{c[2]}W{c[3]}G{c[4]}" for c in LONG_CASES])
def test_attention_parity_long_both_layouts(lf, case, layout, monkeypatch):
    monkeypatch.setenv("LF_ATTN_WAVES", layout)
    B, H, S, W, G, pad = case
    inp = workloads.random_attention_inputs(zlib.crc32(repr(case).encode()) % 100000, B, H, S, W, G, "fp16",
                                            pad_frac=pad)
    _full_compare(lf, inp, W, G, "fp16", f"long-{layout}wave B{B}H{H}S{S}W{W}G{G}")


# unit roundoff of the output / probability type
UNIT = {"fp16": 2.0 ** -11, "bf16": 2.0 ** -8}


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_attention_stress_inputs_std1(lf, dtype):
    # N(0,1) inputs: scores of std ~1 exercise the running-max updates and rescaling;
    # the outputs stay below ~2 in magnitude, so the stated tolerance applies as is
    B, H, S, W, G = 2, 2, 1024, 256, 12
    inp = workloads.random_attention_inputs(77, B, H, S, W, G, dtype, std=1.0,
                                            pad_frac=(0.1, 0.2))
    _full_compare(lf, inp, W, G, dtype, "stress std1")


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_attention_stress_inputs_std2(lf, dtype):
    """N(0,4) inputs: scores of std ~4, so a row's softmax is dominated by a few keys
    and |out| reaches ~8, where one rounding of the output to fp16 is already up to
    2^-11 * 8 ~ 4e-3 (bf16: 3e-2), beyond the absolute tolerance.  The bound is the
    arithmetic's: with u the unit roundoff of the type (fp16 2^-11, bf16 2^-8),
      - the stored output is rounded once:                  <= u |out|;
      - P is rounded to the type before P V, and the row sum is taken from the
        rounded values, so the result is an exact convex combination of the allowed
        v rows whose weights carry a relative error <= 2u / (1 - u):
                                                            <= 2.001 u max|v|;
      - the fp32 accumulations (<= 1e-6 relative) fit in the absolute tolerance.
    Per element: |err| <= TOL + u |ref| + 2.001 u max(|v|, |vg|) of its (b, h)."""
    B, H, S, W, G = 2, 2, 1024, 256, 12
    inp = workloads.random_attention_inputs(78, B, H, S, W, G, dtype, std=2.0,
                                            pad_frac=(0.1, 0.2))
    g = _gpu(inp)
    got = _run(lf, g, W, G).cpu().double().numpy()
    ref = _oracle(inp, W, G)
    u = UNIT[dtype]
    vmax = np.maximum(inp["v"].double().abs().amax(dim=(2, 3)).numpy(),
                      inp["vg"].double().abs().amax(dim=(2, 3)).numpy())[:, :, None, None]
    bound = TOL[dtype] + u * np.abs(ref) + 2.001 * u * vmax
    report(f"stress std2 {dtype}", got, ref, "per-element")
    assert np.all(np.abs(got - ref) <= bound), "error beyond the derived per-element bound"


# ---------------------------------------------------------------- structure
@pytest.mark.parametrize("dtype", ["fp16", "bf16", "fp32"])
def test_identity_values_expose_band_support(lf, dtype):
    # q = qg = 0 and v = vg = I (S = 64 = head_dim): row s is uniform on its allowed
    # keys and exactly 0 elsewhere, so any band / exclusion error shows up as a
    # nonzero entry where the oracle has 0.
    S, W, G = 64, 16, 2
    t = workloads.TORCH_DTYPES[dtype]
    z = torch.zeros(1, 1, S, 64, dtype=t)
    eye = torch.eye(64, dtype=t).view(1, 1, S, 64)
    k = torch.randn(1, 1, S, 64, generator=torch.Generator().manual_seed(0)).to(t)
    lm = torch.ones(1, S, dtype=t)
    gm = torch.full((1, S), -10000.0).to(t)
    gm[0, :G] = 0
    inp = {"q": z, "k": k, "v": eye, "qg": torch.zeros(1, 1, G, 64, dtype=t), "kg": k,
           "vg": eye, "local_mask": lm, "global_mask": gm}
    got = _run(lf, _gpu(inp), W, G).cpu().double().numpy()
    ref = _oracle(inp, W, G)
    assert np.array_equal(got == 0, ref == 0)
    assert np.abs(got - ref).max() <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_ones_values_rows_sum_to_one(lf, dtype):
    B, H, S, W, G = 2, 2, 1024, 256, 9
    inp = workloads.random_attention_inputs(5, B, H, S, W, G, dtype, std=1.0,
                                            pad_frac=(0.1, 0.2))
    inp["v"] = torch.ones_like(inp["v"])
    inp["vg"] = torch.ones_like(inp["vg"])
    got = _run(lf, _gpu(inp), W, G).cpu().double()
    live = inp["local_mask"] == 1
    for b in range(B):
        assert torch.all(got[b][:, live[b]] == 1.0)
        assert torch.all(got[b][:, ~live[b]] == 0.0)


def test_deterministic_and_guard_bands_untouched(lf):
    B, H, S, W, G = 1, 4, 2048, 512, 8
    inp = workloads.random_attention_inputs(9, B, H, S, W, G, "fp16", pad_frac=(0.1, 0.2))
    g = _gpu(inp)
    n = B * H * S * 64
    guard = 4096
    buf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.float16, device="cuda")
    out = buf[guard:guard + n].view(B, H, S, 64)
    _run(lf, g, W, G, out=out)
    first = out.clone()
    _run(lf, g, W, G, out=out)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), out.view(torch.int16))
    assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + n:]).all()


HISTORY_CASES = [
    # B, H, S, W, G, pad: key-split path with helper waves (one and two 16-row passes of
    # their merge), plus the longformer-large shape itself
    (1, 2, 2048, 512, 8, None),
    (2, 2, 1024, 256, 32, (0.05, 0.1)),
    (1, 16, 4096, 512, 8, None),
]


@pytest.mark.parametrize("case", HISTORY_CASES, ids=[f"B{c[0]}H{c[1]}S{c[2]}W{c[3]}G{c[4]}" for c in HISTORY_CASES])
def test_result_independent_of_earlier_calls(lf, case, monkeypatch):
    # A call must not depend on what earlier launches left in LDS, the scratch buffer or
    # the partials: the same inputs give the same bits after calls on other data of the
    # same shape (which run on the same compute units with different values).
    monkeypatch.setenv("LF_ATTN_NO_GWG", "1")
    B, H, S, W, G, pad = case
    mk = lambda seed: _gpu(workloads.random_attention_inputs(seed, B, H, S, W, G, "fp16", pad_frac=pad))
    x, y, z = mk(101), mk(202), mk(303)
    outs = []
    for other in (None, y, z):
        if other is not None:
            _run(lf, other, W, G)
        outs.append(_run(lf, x, W, G))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(outs[0].view(torch.int16), o.view(torch.int16)), "result depends on earlier calls"


@pytest.mark.parametrize("case", [c for c in CASES if 0 < c[4] <= 32 and c[3] >= 160],
                         ids=lambda c: f"B{c[0]}H{c[1]}S{c[2]}W{c[3]}G{c[4]}")
def test_helper_waves_match_band_tile_split(lf, case, monkeypatch):
    # the same launch with the global-row split in helper waves and in the band waves.
    # Local rows: the helper layout takes the global keys inside its first and last band
    # steps instead of in a step of their own, so the same terms are summed in another
    # order under another running-max history (P is rounded to the type relative to that
    # max).  Global rows differ in how the keys are grouped under one running max and in
    # the merge order.  Each path is within u |out| + 2.001 u max|v| of the exact result
    # (the bound derived for the stress test; v for local rows, vg for global rows), so
    # the two are within twice that of each other
    monkeypatch.setenv("LF_ATTN_NO_GWG", "1")
    B, H, S, W, G, pad, ng = case
    inp = workloads.random_attention_inputs(zlib.crc32(repr(case).encode()) % 100000, B, H, S, W, G, "fp16",
                                            pad_frac=pad, n_global=ng)
    g = _gpu(inp)
    a = _run(lf, g, W, G).cpu()
    monkeypatch.setenv("LF_ATTN_NO_HELP", "1")
    b = _run(lf, g, W, G).cpu()
    gm = inp["global_mask"]
    u = UNIT["fp16"]
    vgmax = inp["vg"].double().abs().amax(dim=(2, 3))[:, :, None, None]
    vmax = inp["v"].double().abs().amax(dim=(2, 3))[:, :, None, None]
    for bb in range(B):
        glob = (gm[bb] == 0).numpy()
        for rows, vm, what in ((~glob, vmax, "local"), (glob, vgmax, "global")):
            d = (a[bb][:, rows].double() - b[bb][:, rows].double()).abs()
            bound = 2 * (u * b[bb][:, rows].double().abs() + 2.001 * u * vm[bb])
            print(f"helpers vs band split, b={bb}, {what} rows: "
                  f"max |diff| {float(d.max()) if d.numel() else 0.0:.3e}")
            assert torch.all(d <= bound)


@pytest.mark.parametrize("dtype", ["fp16", "bf16", "fp32"])
def test_preprocessed_entry_point_matches(lf, dtype):
    B, H, S, W, G = 2, 3, 1024, 256, 20
    inp = workloads.random_attention_inputs(11, B, H, S, W, G, dtype, pad_frac=(0.1, 0.2))
    g = _gpu(inp)
    a = _run(lf, g, W, G)
    idx, cnt = lf.init_global_idx(g["global_mask"])
    bias = lf.mask_shift(g["local_mask"])
    b = lf.attn_forward_pre(g["q"], g["k"], g["v"], g["qg"], g["kg"], g["vg"], idx, cnt, bias,
                            W, G)
    torch.cuda.synchronize()
    assert torch.equal(a.cpu().float(), b.cpu().float())


def test_check_masks_detects_violations(lf):
    S, G = 256, 4
    lm = torch.ones(2, S, dtype=torch.float16, device="cuda")
    gm = torch.full((2, S), -10000.0, dtype=torch.float16, device="cuda")
    gm[:, :G] = 0
    lf.check_masks(lm, gm, G)                       # valid
    bad = gm.clone()
    bad[1, 10] = 0                                  # non-leading global
    with pytest.raises(lf.LFError, match="contiguous"):
        lf.check_masks(lm, bad, G)
    with pytest.raises(lf.LFError, match="more than G"):
        lf.check_masks(lm, gm, G - 1)
    bad_l = lm.clone()
    bad_l[0, 3] = 0.5
    with pytest.raises(lf.LFError, match="neither 0 nor 1"):
        lf.check_masks(bad_l, gm, G)
    bad_g = gm.clone()
    bad_g[0, 100] = -5.0
    with pytest.raises(lf.LFError, match="neither 0 nor -10000"):
        lf.check_masks(lm, bad_g, G)


# ---------------------------------------------------------------- full-size workloads
@pytest.mark.parametrize("wl", workloads.ATTN_WORKLOADS[1:], ids=lambda w: w.name)
def test_full_workload_every_element(lf, wl):
    # the longformer-large, padded and long workloads, in the launch configuration the
    # benchmark times, against the oracle over every output element
    inp = workloads.make_attention_inputs(wl)
    g = _gpu(inp)
    out = _run(lf, g, wl.W, wl.G)
    out2 = _run(lf, g, wl.W, wl.G)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), "not deterministic"
    got = out.cpu()
    assert torch.isfinite(got.float()).all()
    _check_padded_zero(got, inp["local_mask"])
    del g, out, out2
    ref = _oracle(inp, wl.W, wl.G)
    err = report(wl.name, got.double().numpy(), ref, TOL[wl.dtype])
    assert err <= TOL[wl.dtype], f"{wl.name}: max abs err {err:.3e}"


@pytest.mark.parametrize("wl", workloads.ATTN_WORKLOADS[1:], ids=lambda w: w.name)
def test_full_workload_other_layout_every_element(lf, wl, monkeypatch):
    # the same workloads in the layout their sequence length does not select (4 waves
    # at S = 4096, 8 waves at S = 16384): both layouts at full size
    monkeypatch.setenv("LF_ATTN_WAVES", "4" if wl.S < 8192 else "8")
    inp = workloads.make_attention_inputs(wl)
    g = _gpu(inp)
    out = _run(lf, g, wl.W, wl.G)
    torch.cuda.synchronize()
    got = out.cpu()
    assert torch.isfinite(got.float()).all()
    _check_padded_zero(got, inp["local_mask"])
    del g, out
    ref = _oracle(inp, wl.W, wl.G)
    err = report(wl.name + " other layout", got.double().numpy(), ref, TOL[wl.dtype])
    assert err <= TOL[wl.dtype], f"{wl.name}: max abs err {err:.3e}"
