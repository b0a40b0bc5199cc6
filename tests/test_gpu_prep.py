"""GPU parity of the preprocessing entry points (bit-exact against the oracle).

[FT-LF] computation flow, preprocessing 1 (global-token indices and count) and 2
(local-mask shift)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DT = workloads.TORCH_DTYPES


@pytest.fixture(scope="module")
def lf():
    import sparse_long_sequence_amd as m
    m.load_library()
    return m


def _idx(lf, gm_cpu):
    idx, cnt = lf.init_global_idx(gm_cpu.cuda())
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy()


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_partition_golden(lf, dtype):
    with open(os.path.join(GOLDEN, "partition_small.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        gm = torch.tensor(c["global_mask"], dtype=DT[dtype])
        idx, cnt = _idx(lf, gm)
        assert idx.tolist() == c["global_idx"]
        assert cnt.tolist() == c["global_count"]


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("B,S", [(1, 1), (3, 7), (2, 1000), (2, 4096), (3, 4097), (2, 16384),
                                 (1, 70000), (2, 300001)])
def test_partition_random_bit_exact(lf, dtype, B, S):
    # S = 4097 and 300001: rows that start off a 16-byte boundary (the count of
    # earlier flags takes narrow loads); 70000 and 300001: several passes per
    # workgroup, 300001: more than 64 chunks of 1024 positions
    rng = np.random.default_rng(B * 100003 + S)
    dens = rng.uniform(0, 1, size=(B, 1))
    flags = rng.uniform(size=(B, S)) < dens
    gm = torch.tensor(np.where(flags, 0.0, -10000.0), dtype=DT[dtype])
    idx, cnt = _idx(lf, gm)
    ridx, rcnt = oracle.global_partition(gm)
    assert np.array_equal(cnt, rcnt)
    assert np.array_equal(idx, ridx)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_partition_extremes_and_signed_zero(lf, dtype):
    S = 5000
    for gm in (torch.zeros(2, S), torch.full((2, S), -10000.0), -torch.zeros(1, S)):
        gm = gm.to(DT[dtype])
        idx, cnt = _idx(lf, gm)
        ridx, rcnt = oracle.global_partition(gm)
        assert np.array_equal(idx, ridx) and np.array_equal(cnt, rcnt)


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_partition_workload_masks(lf, dtype):
    for wl in workloads.ATTN_WORKLOADS:
        rng = np.random.default_rng(wl.seed)
        _, gm = workloads.make_masks(rng, wl.B, wl.S, wl.G, dtype, wl.pad_frac)
        idx, cnt = _idx(lf, gm)
        ridx, rcnt = oracle.global_partition(gm)
        assert np.array_equal(idx, ridx) and np.array_equal(cnt, rcnt)


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_mask_shift_golden(lf, dtype):
    with open(os.path.join(GOLDEN, "mask_shift_values.json")) as f:
        cases = json.load(f)["cases"][dtype]
    m = torch.tensor([[c[0] for c in cases]], dtype=DT[dtype])
    got = lf.mask_shift(m.cuda()).cpu()
    assert got.dtype == DT[dtype]
    assert got.to(torch.float64).tolist()[0] == [c[1] for c in cases]


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("B,S", [(1, 1), (3, 13), (4, 4096), (2, 16384), (1, 100003)])
def test_mask_shift_bit_exact(lf, dtype, B, S):
    rng = np.random.default_rng(S)
    vals = np.where(rng.uniform(size=(B, S)) < 0.5, rng.uniform(-2, 2, size=(B, S)),
                    rng.integers(0, 2, size=(B, S)).astype(np.float64))
    m = torch.tensor(vals, dtype=DT[dtype])
    got = lf.mask_shift(m.cuda()).cpu()
    ref = oracle.mask_shift(m, dtype)
    assert torch.equal(got.view(torch.int16 if dtype != "fp32" else torch.int32),
                       ref.view(torch.int16 if dtype != "fp32" else torch.int32))
