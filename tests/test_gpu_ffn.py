"""GPU parity of the FFN block (lf_ffn_block): the two-GEMM path the layer runs and the
fused one-kernel path, against the float64 oracle's ffn_block.

[FT-LF] computation flow, per-layer step 6: y = LN(resid + GELU(h W1^T + b1) W2^T + b2).
The fused path follows the operator fusion of the page "300%加速！PaddleNLP FastFFN如何让
大模型训练"飞"起来" (section "技术原理深入解析", item 1): the GELU output never goes to
global memory.  Tolerances as for the layer output (tests/test_gpu_layer.py): fp16 3e-3,
bf16 2.5e-2 + 2^-8 |ref|, fp32 1e-4; both paths round the intermediate to the input
type, so they meet the same bar and agree with each other to twice it."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import report

pytestmark = pytest.mark.gpu

TOL = {"fp16": 3e-3, "bf16": 2.5e-2, "fp32": 1e-4}


@pytest.fixture(scope="module")
def lf():
    import sparse_long_sequence_amd as m
    m.load_library()
    return m


def _inputs(seed, M, D, F, dtype):
    rng = np.random.default_rng(seed)
    w = workloads.random_layer_params(rng, D, F, dtype, w_std=0.05, b_std=0.02, ln_jitter=0.1)
    resid = torch.from_numpy(rng.standard_normal((M, D))).to(torch.float32)
    h = resid.to(workloads.TORCH_DTYPES[dtype])   # the GEMM copy of the residual stream
    return h, resid, w


def _run(lf, h, resid, w, fused):
    g = {n: w[n].cuda() for n in ("w_ffn1", "b_ffn1", "w_ffn2", "b_ffn2", "ln2_g", "ln2_b")}
    y = lf.ffn_block(h.cuda(), resid.cuda(), g["w_ffn1"], g["b_ffn1"], g["w_ffn2"], g["b_ffn2"],
                     g["ln2_g"], g["ln2_b"], fused=fused)
    torch.cuda.synchronize()
    return y.cpu()


def _oracle(h, resid, w, rows=None):
    if rows is not None:
        h, resid = h[rows], resid[rows]
    return oracle.ffn_block(h, resid, w["w_ffn1"], w["b_ffn1"], w["w_ffn2"], w["b_ffn2"],
                            w["ln2_g"], w["ln2_b"])


def _check(got, ref, dtype, case="ffn"):
    report(f"{case} {dtype}", got.double().numpy(), ref, TOL[dtype] if dtype != "bf16" else "per-element")
    err = np.abs(got.double().numpy() - ref)
    tol = TOL[dtype] + (2.0 ** -8 * np.abs(ref) if dtype == "bf16" else 0.0)
    assert np.all(err <= tol), f"max abs err {err.max():.3e}"


@pytest.mark.parametrize("fused", [False, True], ids=["two_gemm", "fused"])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("case", [
    (100, 256, 512),    # ragged rows (not a multiple of 32 or 128)
    (64, 512, 1024),
    (70, 768, 256),     # one F chunk per slice after the split
    (96, 1024, 2048),
], ids=lambda c: f"M{c[0]}_D{c[1]}_F{c[2]}")
def test_ffn_block_vs_oracle(lf, case, dtype, fused):
    M, D, F = case
    h, resid, w = _inputs(500 + M + D, M, D, F, dtype)
    got = _run(lf, h, resid, w, fused)
    assert torch.isfinite(got.float()).all()
    _check(got, _oracle(h, resid, w), dtype)


def test_ffn_block_fp32_two_gemm(lf):
    h, resid, w = _inputs(601, 80, 256, 512, "fp32")
    _check(_run(lf, h, resid, w, False), _oracle(h, resid, w), "fp32")


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_fused_and_two_gemm_agree_and_fused_is_deterministic(lf, dtype):
    h, resid, w = _inputs(602, 200, 512, 1024, dtype)
    a = _run(lf, h, resid, w, True)
    a2 = _run(lf, h, resid, w, True)
    b = _run(lf, h, resid, w, False)
    assert torch.equal(a.view(torch.int16), a2.view(torch.int16)), "fused path not deterministic"
    err = (a.double() - b.double()).abs()
    tol = 2 * TOL[dtype] + (2.0 ** -7 * b.double().abs() if dtype == "bf16" else 0.0)
    assert bool((err <= tol).all()), f"max |fused - two_gemm| {err.max().item():.3e}"


@pytest.mark.parametrize("fused", [False, True], ids=["two_gemm", "fused"])
@pytest.mark.parametrize("M,dtype", [(8192, "fp16"), (1024, "fp16"), (8192, "bf16")],
                         ids=["layer_rows_fp16", "stack_rows_fp16", "layer_rows_bf16"])
def test_ffn_block_full_size_every_element(lf, M, dtype, fused):
    # the layer's FFN (M = 2 x 4096 rows, D 1024, F 4096) and the stack benchmark's
    # (M = 1024: the fused path splits F over workgroups), every output element
    D, F = 1024, 4096
    h, resid, w = _inputs(603 + M, M, D, F, dtype)
    got = _run(lf, h, resid, w, fused)
    assert torch.isfinite(got.float()).all()
    _check(got, _oracle(h, resid, w), dtype, f"ffn M{M} {'fused' if fused else 'two-GEMM'}")
