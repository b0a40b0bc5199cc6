"""GPU tests of the encoder stack (preprocessing once, then the layer loop).

[FT-LF] computation flow: the preprocessing list (global-token index, mask shift)
runs once and every layer's attention reads its result.  The stack must equal the
single-layer entry point applied layer after layer (bit for bit: same kernels; the
attention's preprocessed-mask mode computes exactly what its raw-mask mode does), and
its last layer must match the float64 oracle given the same input (fp16 3e-3)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import report

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lf():
    import sparse_long_sequence_amd as m
    m.load_library()
    return m


def _setup(seed, B, S, D, H, F, G, L, dtype, pad=None):
    rng = np.random.default_rng(seed)
    layers = [workloads.random_layer_params(rng, D, F, dtype, w_std=0.05, b_std=0.02,
                                            ln_jitter=0.1) for _ in range(L)]
    x = torch.from_numpy(rng.standard_normal((B, S, D))).to(workloads.TORCH_DTYPES[dtype])
    lm, gm = workloads.make_masks(rng, B, S, G, dtype, pad, None)
    return x, layers, lm, gm


@pytest.mark.parametrize("dtype", ["fp16", "bf16", "fp32"])
@pytest.mark.parametrize("case", [(1, 512, 256, 4, 512, 128, 8, None, 3),
                                  (2, 384, 512, 8, 1024, 64, 0, (0.1, 0.25), 2)],
                         ids=["B1_S512_G8_L3", "B2_S384_G0_pad_L2"])
def test_stack_equals_layer_after_layer(lf, dtype, case):
    B, S, D, H, F, W, G, pad, L = case
    x, layers, lm, gm = _setup(21 + L, B, S, D, H, F, G, L, dtype, pad)
    xg, lmg, gmg = x.cuda(), lm.cuda(), gm.cuda()
    wg = [{n: t.cuda() for n, t in w.items()} for w in layers]
    y = lf.encoder_forward(xg, wg, lmg, gmg, H, W, G)
    cur = xg
    for w in wg:
        cur = lf.encoder_layer(cur, w, lmg, gmg, H, W, G)
    torch.cuda.synchronize()
    bits = torch.int32 if dtype == "fp32" else torch.int16
    assert torch.equal(y.view(bits), cur.view(bits))
    assert torch.equal(x, xg.cpu()), "the stack must not write its input"


def test_stack_last_layer_matches_oracle(lf):
    B, S, D, H, F, W, G, L = 1, 512, 256, 4, 512, 128, 8, 2
    x, layers, lm, gm = _setup(31, B, S, D, H, F, G, L, "fp16")
    xg, lmg, gmg = x.cuda(), lm.cuda(), gm.cuda()
    wg = [{n: t.cuda() for n, t in w.items()} for w in layers]
    y1 = lf.encoder_layer(xg, wg[0], lmg, gmg, H, W, G)
    y = lf.encoder_forward(xg, wg, lmg, gmg, H, W, G)
    torch.cuda.synchronize()
    ref = oracle.encoder_layer(y1.cpu(), layers[1], lm, gm, H, W, G)
    err = report("stack S512 D256 last layer fp16", y.cpu().double().numpy(), ref, 3e-3)
    assert err <= 3e-3, f"max abs err {err:.3e}"


@pytest.mark.parametrize("split_path", [False, True], ids=["default", "split_path"])
def test_stack_benchmark_shape_every_layer_vs_oracle(lf, split_path, monkeypatch):
    """The encoder stack at the shape the pages benchmark ([FT-LF] section "性能基准：FP32
    与 FP16": 16 heads x 64, intermediate 4096, window 512; batch 1, sequence 1024) with
    16 leading global tokens and 3 layers.  This shape takes the kernel paths of small
    grids: 64 x 128 GEMM tiles, the output projection and FFN2 split over K with the
    partial sums reduced in the LayerNorm kernel, and the global rows in workgroups of
    their own (split_path: LF_ATTN_NO_GWG=1, the key-split path instead).  Layer l of
    the stack is checked over every element against the oracle's layer applied to the
    stack's own output after l - 1 layers."""
    if split_path:
        monkeypatch.setenv("LF_ATTN_NO_GWG", "1")
    B, S, D, H, F, W, G, L = 1, 1024, 1024, 16, 4096, 512, 16, 3
    rng = np.random.default_rng(41)
    layers = [workloads.random_layer_params(rng, D, F, "fp16", w_std=0.02, b_std=0.02,
                                            ln_jitter=0.1) for _ in range(L)]
    x = torch.from_numpy(rng.standard_normal((B, S, D))).to(torch.float16)
    lm, gm = workloads.make_masks(rng, B, S, G, "fp16")
    xg, lmg, gmg = x.cuda(), lm.cuda(), gm.cuda()
    wg = [{n: t.cuda() for n, t in w.items()} for w in layers]
    prev = x
    for l in range(L):
        y = lf.encoder_forward(xg, wg[:l + 1], lmg, gmg, H, W, G)
        torch.cuda.synchronize()
        got = y.cpu()
        assert torch.isfinite(got.float()).all()
        ref = oracle.encoder_layer(prev, layers[l], lm, gm, H, W, G)
        err = report(f"stack B1 S1024 D1024 F4096 layer {l}{' split' if split_path else ''}",
                     got.double().numpy(), ref, 3e-3)
        assert err <= 3e-3, f"layer {l}: max abs err {err:.3e}"
        prev = got


def test_stack_rejects_zero_layers(lf):
    x, layers, lm, gm = _setup(1, 1, 256, 256, 4, 256, 4, 1, "fp16")
    with pytest.raises(ValueError):
        lf.encoder_forward(x.cuda(), [], lm.cuda(), gm.cuda(), 4, 64, 4)
