"""CPU-side checks of the C ABI: the library loads, exports every symbol the header
declares, and rejects bad arguments on the host before touching the GPU."""
import ctypes
import os
import re

import pytest

import sparse_long_sequence_amd as lf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lf.h")

INVALID = 1
UNSUPPORTED = 2


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lf_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lf.library_path()):
        pytest.skip("liblf.so not built")
    return lf.load_library()


def test_header_declares_expected_entry_points():
    assert set(_declared()) == set(lf.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert lib.lf_status_string(0) == b"ok"
    assert lib.lf_status_string(1) == b"invalid argument"
    assert lib.lf_status_string(4) == b"precondition violated"


def _fake(n=1):
    return ctypes.c_void_p(0x1000)


ATTN_ENTRIES = ["lf_attn_forward", "lf_attn_forward_any_globals"]


def _attn(lib, dtype=1, B=1, H=2, S=64, W=16, G=2, null=None, entry="lf_attn_forward"):
    p = {n: _fake() for n in ("q", "k", "v", "qg", "kg", "vg", "lm", "gm", "out")}
    if null:
        p[null] = None
    return getattr(lib, entry)(dtype, p["q"], p["k"], p["v"], p["qg"], p["kg"], p["vg"], p["lm"],
                               p["gm"], B, H, S, W, G, p["out"], None)


@pytest.mark.parametrize("kw,msg", [
    (dict(S=60, W=16), "S % W"),          # hard constraint 1: divisibility
    (dict(S=16, W=16), "S must be >= 2*W"),
    (dict(G=17, W=16), "G must satisfy"),  # hard constraint 3
    (dict(G=-1), "G must satisfy"),
    (dict(W=15, S=60), "even"),
    (dict(W=0), "even"),
    (dict(B=0), ">= 1"),
    (dict(H=0), ">= 1"),
    (dict(dtype=7), "dtype"),
])
@pytest.mark.parametrize("entry", ATTN_ENTRIES)
def test_attn_shape_rules_rejected_on_host(lib, kw, msg, entry):
    assert _attn(lib, entry=entry, **kw) == INVALID
    assert msg in lib.lf_last_error().decode()


@pytest.mark.parametrize("name", ["q", "k", "v", "kg", "vg", "lm", "gm", "out", "qg"])
@pytest.mark.parametrize("entry", ATTN_ENTRIES)
def test_attn_null_pointers_rejected(lib, name, entry):
    assert _attn(lib, null=name, entry=entry) == INVALID
    assert "null pointer" in lib.lf_last_error().decode()


def test_qg_may_be_null_without_globals(lib):
    # G == 0 and qg NULL passes validation; a NULL k still fails, proving no launch happened
    p = _fake()
    st = lib.lf_attn_forward(1, p, None, p, None, p, p, p, p, 1, 1, 64, 16, 0, p, None)
    assert st == INVALID and "k" in lib.lf_last_error().decode()


def test_workspace_size_query(lib):
    assert lib.lf_attn_workspace_bytes(1, 1, 16, 4096, 512, 8) > 0
    assert lib.lf_attn_workspace_bytes(1, 1, 16, 4095, 512, 8) == 0   # bad shape -> 0
    assert lib.lf_attn_workspace_bytes(1, 1, 16, 4096, 512, 8) % 256 == 0


def test_pre_rejects_small_or_misaligned_workspace(lib):
    p = _fake()
    need = lib.lf_attn_workspace_bytes(1, 1, 2, 64, 16, 2)
    st = lib.lf_attn_forward_pre(1, p, p, p, p, p, p, p, p, p, 1, 2, 64, 16, 2, p, p, need - 1,
                                 None)
    assert st == INVALID and "too small" in lib.lf_last_error().decode()
    st = lib.lf_attn_forward_pre(1, p, p, p, p, p, p, p, p, p, 1, 2, 64, 16, 2, p,
                                 ctypes.c_void_p(0x1008), need, None)
    assert st == INVALID and "aligned" in lib.lf_last_error().decode()


def test_prep_entry_points_validate(lib):
    p = _fake()
    assert lib.lf_init_global_idx(1, p, 0, 8, p, p, None) == INVALID
    assert lib.lf_init_global_idx(1, None, 1, 8, p, p, None) == INVALID
    assert lib.lf_init_global_idx(5, p, 1, 8, p, p, None) == INVALID
    assert lib.lf_mask_shift(1, p, 1, 0, p, None) == INVALID
    assert lib.lf_mask_shift(1, p, 1, 8, None, None) == INVALID
    assert lib.lf_check_masks(1, None, p, 1, 8, 2, None) == INVALID


def test_python_binding_refuses_cpu_tensors(lib):
    import torch
    x = torch.zeros(1, 8, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        lf.mask_shift(x)


def test_ffn_block_validates_on_host(lib):
    # [FT-LF] per-layer step 6 on its own; the fused mode covers fp16 / bf16 and
    # D <= 1024 only (no GPU work happens for any of these calls)
    p = _fake()
    assert lib.lf_ffn_block_workspace_bytes(1, 8192, 1024, 4096, 0) > 0
    assert lib.lf_ffn_block_workspace_bytes(1, 8192, 1024, 4096, 1) > 0
    assert lib.lf_ffn_block_workspace_bytes(1, 8192, 1000, 4096, 0) == 0    # D % 128
    assert lib.lf_ffn_block_workspace_bytes(0, 8192, 1024, 4096, 1) == 0    # fp32 fused
    assert lib.lf_ffn_block_workspace_bytes(1, 64, 2048, 4096, 1) == 0      # D > 1024 fused
    assert lib.lf_ffn_block_workspace_bytes(1, 64, 2048, 4096, 0) > 0
    args = lambda dt, M, D, F, fused, ws: (dt, p, p, p, p, p, p, p, p, M, D, F,
                                           ctypes.c_float(1e-5), fused, p, p, ws, None)
    need = lib.lf_ffn_block_workspace_bytes(1, 64, 256, 512, 1)
    assert lib.lf_ffn_block(*args(0, 64, 256, 512, 1, 1 << 30)) == UNSUPPORTED
    assert "fp16 / bf16" in lib.lf_last_error().decode()
    assert lib.lf_ffn_block(*args(1, 64, 256, 500, 1, 1 << 30)) == INVALID
    assert lib.lf_ffn_block(*args(1, 0, 256, 512, 0, 1 << 30)) == INVALID
    assert lib.lf_ffn_block(*args(1, 64, 256, 512, 1, need - 1)) == INVALID
    assert "too small" in lib.lf_last_error().decode()
    st = lib.lf_ffn_block(1, p, None, p, p, p, p, p, p, 64, 256, 512, ctypes.c_float(1e-5), 0,
                          p, p, 1 << 30, None)
    assert st == INVALID and "resid" in lib.lf_last_error().decode()
