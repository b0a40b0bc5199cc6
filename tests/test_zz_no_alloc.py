"""lf_attn_forward_noalloc (the entry point for callers that cannot allocate device
memory) against lf_attn_forward, through the C ABI.

Both run the same kernels with the same work split, so the outputs must agree bit for
bit.  Two calls in a row on the shared scratch array, the second with a smaller input:
the second must not see anything the first left behind.  A shape whose scratch exceeds
the array's capacity is rejected on the host with the output untouched."""
import ctypes

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import sparse_long_sequence_amd as m
    lib = m.load_library()
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.lf_attn_forward_noalloc.argtypes = [I, P, P, P, P, P, P, P, P, I, I, I, I, I, P, P]
    lib.lf_attn_forward_noalloc.restype = I
    lib.lf_attn_forward_noalloc_max_scratch.argtypes = []
    lib.lf_attn_forward_noalloc_max_scratch.restype = ctypes.c_size_t
    return lib


def _call(lib, entry, g, W, G, out):
    import sparse_long_sequence_amd as m
    B, H, S, _ = g["q"].shape
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return entry(m.dtype_code(g["q"].dtype), p(g["q"]), p(g["k"]), p(g["v"]), p(g["qg"]),
                 p(g["kg"]), p(g["vg"]), p(g["local_mask"]), p(g["global_mask"]), B, H, S, W, G,
                 p(out), st)


def _pair(lib, seed, B, H, S, W, G, dtype, pad):
    inp = workloads.random_attention_inputs(seed, B, H, S, W, G, dtype, pad_frac=pad)
    g = {n: t.cuda() for n, t in inp.items()}
    ref = torch.empty_like(g["q"])
    got = torch.full_like(g["q"], float("nan"))
    assert _call(lib, lib.lf_attn_forward, g, W, G, ref) == 0
    assert _call(lib, lib.lf_attn_forward_noalloc, g, W, G, got) == 0
    torch.cuda.synchronize()
    bits = torch.int32 if dtype == "fp32" else torch.int16
    return torch.equal(ref.view(bits), got.view(bits))


@pytest.mark.parametrize("dtype", ["fp16", "bf16", "fp32"])
def test_noalloc_matches_attn_forward_twice_second_smaller(lib, dtype):
    # first: the longformer-large shape (its grid takes the key-split path: tickets and
    # partials in the array); second: a smaller padded problem with more global rows
    if dtype == "fp32":
        first, second = (1, 2, 1024, 256, 8, None), (1, 1, 512, 128, 3, (0.1, 0.2))
    else:
        first, second = (1, 16, 4096, 512, 8, None), (2, 3, 1024, 256, 20, (0.1, 0.25))
    assert _pair(lib, 5, *first[:5], dtype, first[5])
    assert _pair(lib, 6, *second[:5], dtype, second[5])


def test_noalloc_split_path_on_small_grid(lib, monkeypatch):
    # the key-split path (tickets in the array) on a grid that would otherwise take the
    # per-(batch, head) global-row workgroups
    monkeypatch.setenv("LF_ATTN_NO_GWG", "1")
    assert _pair(lib, 7, 2, 2, 1024, 128, 33, "fp16", (0.05, 0.1))
    assert _pair(lib, 8, 1, 2, 512, 128, 5, "fp16", None)


def test_noalloc_rejects_a_shape_beyond_its_scratch(lib):
    import sparse_long_sequence_amd as m
    # partials of 4 x 16 heads x 32 splits x 512 global rows exceed the array
    B, H, S, W, G = 4, 16, 16384, 512, 512
    cap = lib.lf_attn_forward_noalloc_max_scratch()
    need = B * H * 32 * G * 68 * 4
    assert need > cap
    t = torch.zeros(1, dtype=torch.float16, device="cuda")
    out = torch.full((8,), 7.0, dtype=torch.float16, device="cuda")
    p = ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.lf_attn_forward_noalloc(m.dtype_code(torch.float16), p, p, p, p, p, p, p, p, B, H, S,
                                     W, G, ctypes.c_void_p(out.data_ptr()), st)
    assert rc == 2   # LF_ERR_UNSUPPORTED, nothing enqueued
    assert b"scratch" in lib.lf_last_error()
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
