"""Longformer band + global attention for MI355X (gfx950): Python binding of liblf.so.

Argument marshalling only: every step runs in the library's HIP kernels.  Tensors
must already live on the GPU; there is no CPU fallback, and calling any function
without the built library raises.

Citations in this package refer to the page "FasterTransformer Longformer 推理加速
实践：PyTorch 集成、输入约束与端到端性能解析" ([FT-LF]).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["LFError", "library_path", "load_library", "init_global_idx", "mask_shift",
           "attn_forward", "attn_forward_any_globals", "attn_forward_pre", "attn_workspace_bytes",
           "attn_forward_noalloc",
           "check_masks",
           "encoder_layer", "encoder_layer_workspace_bytes", "encoder_forward",
           "encoder_forward_workspace_bytes", "LAYER_WEIGHT_FIELDS",
           "ffn_block", "ffn_block_workspace_bytes",
           "kernel_timing_start", "kernel_timing_stop", "release_stream_scratch",
           "EXPORTED_SYMBOLS", "dtype_code"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liblf.so")
_lib = None

LF_OK = 0
_DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}

LAYER_WEIGHT_FIELDS = ["w_proj", "b_proj", "w_qg", "b_qg", "w_o", "b_o", "ln1_g", "ln1_b",
                       "w_ffn1", "b_ffn1", "w_ffn2", "b_ffn2", "ln2_g", "ln2_b"]

EXPORTED_SYMBOLS = ["lf_init_global_idx", "lf_mask_shift", "lf_attn_forward",
                    "lf_attn_forward_noalloc", "lf_attn_forward_noalloc_max_scratch",
                    "lf_attn_forward_any_globals",
                    "lf_attn_workspace_bytes", "lf_attn_forward_pre", "lf_check_masks",
                    "lf_encoder_layer_workspace_bytes", "lf_encoder_layer",
                    "lf_encoder_layer_any_globals",
                    "lf_encoder_forward_workspace_bytes", "lf_encoder_forward",
                    "lf_encoder_forward_any_globals",
                    "lf_ffn_block_workspace_bytes", "lf_ffn_block",
                    "lf_kernel_timing_start", "lf_kernel_timing_stop",
                    "lf_release_stream_scratch",
                    "lf_status_string", "lf_last_error"]


class LFError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"lf status {status}: {msg}")
        self.status = status


class _LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_WEIGHT_FIELDS]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load liblf.so (built by __graft_entry__.build()); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"HIP library not built: {_LIB_PATH} is missing "
                           "(run __graft_entry__.build())")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.lf_init_global_idx.argtypes = [I, P, I, I, P, P, P]
    lib.lf_mask_shift.argtypes = [I, P, I, I, P, P]
    lib.lf_attn_forward.argtypes = [I, P, P, P, P, P, P, P, P, I, I, I, I, I, P, P]
    lib.lf_attn_forward_any_globals.argtypes = [I, P, P, P, P, P, P, P, P, I, I, I, I, I, P, P]
    lib.lf_attn_forward_noalloc.argtypes = [I, P, P, P, P, P, P, P, P, I, I, I, I, I, P, P]
    lib.lf_attn_forward_noalloc_max_scratch.argtypes = []
    lib.lf_attn_forward_noalloc_max_scratch.restype = S
    lib.lf_attn_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.lf_attn_workspace_bytes.restype = S
    lib.lf_attn_forward_pre.argtypes = [I, P, P, P, P, P, P, P, P, P, I, I, I, I, I, P, P, S, P]
    lib.lf_check_masks.argtypes = [I, P, P, I, I, I, P]
    lib.lf_encoder_layer_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I]
    lib.lf_encoder_layer_workspace_bytes.restype = S
    lib.lf_encoder_layer.argtypes = [I, ctypes.POINTER(_LayerWeights), P, P, P, I, I, I, I, I,
                                     I, I, ctypes.c_float, ctypes.c_float, P, P, S, P]
    lib.lf_encoder_layer_any_globals.argtypes = lib.lf_encoder_layer.argtypes
    lib.lf_encoder_forward_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I]
    lib.lf_encoder_forward_workspace_bytes.restype = S
    lib.lf_encoder_forward.argtypes = [I, ctypes.POINTER(_LayerWeights), I, P, P, P, I, I, I, I,
                                       I, I, I, ctypes.c_float, ctypes.c_float, P, P, S, P]
    lib.lf_encoder_forward_any_globals.argtypes = lib.lf_encoder_forward.argtypes
    lib.lf_ffn_block_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.lf_ffn_block_workspace_bytes.restype = S
    lib.lf_ffn_block.argtypes = [I, P, P, P, P, P, P, P, P, I, I, I, ctypes.c_float, I, P, P, S,
                                 P]
    lib.lf_release_stream_scratch.argtypes = [P]
    lib.lf_kernel_timing_start.argtypes = [I]
    lib.lf_kernel_timing_stop.argtypes = [ctypes.POINTER(ctypes.c_int),
                                          ctypes.POINTER(ctypes.c_double)]
    lib.lf_status_string.argtypes = [I]
    lib.lf_status_string.restype = ctypes.c_char_p
    lib.lf_last_error.argtypes = []
    lib.lf_last_error.restype = ctypes.c_char_p
    for name in ("lf_init_global_idx", "lf_mask_shift", "lf_attn_forward",
                 "lf_attn_forward_any_globals", "lf_attn_forward_noalloc",
                 "lf_attn_forward_pre", "lf_check_masks", "lf_encoder_layer",
                 "lf_encoder_forward", "lf_encoder_layer_any_globals",
                 "lf_encoder_forward_any_globals", "lf_ffn_block",
                 "lf_kernel_timing_start", "lf_kernel_timing_stop", "lf_release_stream_scratch"):
        getattr(lib, name).restype = I
    _lib = lib
    return lib


def _check(status: int):
    if status != LF_OK:
        lib = load_library()
        raise LFError(status, lib.lf_last_error().decode())


def dtype_code(t: torch.dtype) -> int:
    if t not in _DTYPE_CODE:
        raise TypeError(f"unsupported dtype {t}")
    return _DTYPE_CODE[t]


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU (no CPU fallback)")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors must be on one device")
    return dev


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def init_global_idx(global_mask: torch.Tensor, global_idx=None, global_count=None):
    """[FT-LF computation flow, preprocessing 1] -> (global_idx int32 [B,S], count int32 [B])."""
    lib = load_library()
    dev = _dev(global_mask)
    B, S = global_mask.shape
    if global_idx is None:
        global_idx = torch.empty(B, S, dtype=torch.int32, device=dev)
    if global_count is None:
        global_count = torch.empty(B, dtype=torch.int32, device=dev)
    _dev(global_idx, global_count)
    _check(lib.lf_init_global_idx(dtype_code(global_mask.dtype), _ptr(global_mask), B, S,
                                  _ptr(global_idx), _ptr(global_count), _stream(dev)))
    return global_idx, global_count


def mask_shift(local_mask: torch.Tensor, out=None):
    """[FT-LF computation flow, preprocessing 2] -> fma(mask, 10000, -10000) in mask dtype."""
    lib = load_library()
    dev = _dev(local_mask)
    B, S = local_mask.shape
    if out is None:
        out = torch.empty_like(local_mask)
    _dev(out)
    _check(lib.lf_mask_shift(dtype_code(local_mask.dtype), _ptr(local_mask), B, S, _ptr(out),
                             _stream(dev)))
    return out


def _attn_shapes(q, qg, W, G):
    B, H, S, D = q.shape
    if D != 64:
        raise ValueError("head_dim must be 64")
    if qg is not None and tuple(qg.shape) != (B, H, G, 64):
        raise ValueError(f"qg must be [B,H,G,64] = {(B, H, G, 64)}, got {tuple(qg.shape)}")
    return B, H, S


def attn_forward(q, k, v, qg, kg, vg, local_mask, global_mask, W: int, G: int, out=None):
    """[FT-LF computation flow, per-layer steps 3-4] band + global attention -> out [B,H,S,64]."""
    lib = load_library()
    dev = _dev(q, k, v, qg, kg, vg, local_mask, global_mask)
    B, H, S = _attn_shapes(q, qg, W, G)
    for t in (k, v, kg, vg):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v, kg, vg must share shape and dtype")
    if out is None:
        out = torch.empty_like(q)
    _dev(out)
    _check(lib.lf_attn_forward(dtype_code(q.dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(qg),
                               _ptr(kg), _ptr(vg), _ptr(local_mask), _ptr(global_mask),
                               B, H, S, W, G, _ptr(out), _stream(dev)))
    return out


def attn_forward_any_globals(q, k, v, qg, kg, vg, local_mask, global_mask, W: int, G: int,
                             out=None):
    """Band + global attention with the global tokens at any positions -> out [B,H,S,64]."""
    lib = load_library()
    dev = _dev(q, k, v, qg, kg, vg, local_mask, global_mask)
    B, H, S = _attn_shapes(q, qg, W, G)
    for t in (k, v, kg, vg):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v, kg, vg must share shape and dtype")
    if out is None:
        out = torch.empty_like(q)
    _dev(out)
    _check(lib.lf_attn_forward_any_globals(dtype_code(q.dtype), _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(qg), _ptr(kg), _ptr(vg), _ptr(local_mask),
                                           _ptr(global_mask), B, H, S, W, G, _ptr(out),
                                           _stream(dev)))
    return out


def attn_forward_noalloc(q, k, v, qg, kg, vg, local_mask, global_mask, W: int, G: int, out):
    """lf_attn_forward_noalloc: the attention with its scratch in the library's static
    device array (no allocation inside the library; `out` must be given)."""
    lib = load_library()
    dev = _dev(q, k, v, qg, kg, vg, local_mask, global_mask, out)
    B, H, S = _attn_shapes(q, qg, W, G)
    _check(lib.lf_attn_forward_noalloc(dtype_code(q.dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(qg),
                                       _ptr(kg), _ptr(vg), _ptr(local_mask), _ptr(global_mask),
                                       B, H, S, W, G, _ptr(out), _stream(dev)))
    return out


def attn_workspace_bytes(dtype: torch.dtype, B, H, S, W, G) -> int:
    return int(load_library().lf_attn_workspace_bytes(dtype_code(dtype), B, H, S, W, G))


def attn_forward_pre(q, k, v, qg, kg, vg, global_idx, global_count, local_bias, W: int, G: int,
                     out=None, workspace=None):
    """Attention on preprocessed masks; allocates nothing inside the library."""
    lib = load_library()
    dev = _dev(q, k, v, qg, kg, vg, global_idx, global_count, local_bias)
    B, H, S = _attn_shapes(q, qg, W, G)
    if out is None:
        out = torch.empty_like(q)
    nbytes = attn_workspace_bytes(q.dtype, B, H, S, W, G)
    if workspace is None:
        # the leading split tickets must start at zero; the library leaves them zero
        workspace = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
    _dev(out, workspace)
    _check(lib.lf_attn_forward_pre(dtype_code(q.dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(qg),
                                   _ptr(kg), _ptr(vg), _ptr(global_idx), _ptr(global_count),
                                   _ptr(local_bias), B, H, S, W, G, _ptr(out), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(dev)))
    return out


def release_stream_scratch(stream=None):
    """Free the scratch buffer the attention entry points keep for `stream` (default: the
    current stream of the current device); stream-ordered, no sync."""
    st = stream if stream is not None else torch.cuda.current_stream()
    _check(load_library().lf_release_stream_scratch(ctypes.c_void_p(st.cuda_stream)))


def kernel_timing_start(capacity: int):
    """Record HIP events around the main attention kernel of the next `capacity` calls."""
    _check(load_library().lf_kernel_timing_start(capacity))


def kernel_timing_stop():
    """-> (launches, total_ms) of the main attention kernel since kernel_timing_start."""
    n = ctypes.c_int(0)
    ms = ctypes.c_double(0.0)
    _check(load_library().lf_kernel_timing_stop(ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def check_masks(local_mask, global_mask, G: int):
    """Synchronous precondition check; raises LFError(status 4) on a violation."""
    lib = load_library()
    dev = _dev(local_mask, global_mask)
    B, S = local_mask.shape
    _check(lib.lf_check_masks(dtype_code(local_mask.dtype), _ptr(local_mask), _ptr(global_mask),
                              B, S, G, _stream(dev)))


def encoder_layer_workspace_bytes(dtype, B, S, hidden, H, ffn, W, G) -> int:
    return int(load_library().lf_encoder_layer_workspace_bytes(dtype_code(dtype), B, S, hidden, H,
                                                               ffn, W, G))


def encoder_layer(x, weights: dict, local_mask, global_mask, H: int, W: int, G: int,
                  attn_scale: float = 0.125, ln_eps: float = 1e-5, out=None, workspace=None,
                  any_globals: bool = False):
    """[FT-LF computation flow, per-layer steps 1-6] one encoder layer -> y [B,S,hidden].

    any_globals: the global tokens may sit at any positions (lf_encoder_layer_any_globals).
    """
    lib = load_library()
    entry = lib.lf_encoder_layer_any_globals if any_globals else lib.lf_encoder_layer
    ws = [weights[n] for n in LAYER_WEIGHT_FIELDS]
    dev = _dev(x, local_mask, global_mask, *ws)
    B, S, D = x.shape
    F = weights["w_ffn1"].shape[0]
    if out is None:
        out = torch.empty_like(x)
    nbytes = encoder_layer_workspace_bytes(x.dtype, B, S, D, H, F, W, G)
    if workspace is None:
        # the leading split tickets must start at zero; the library leaves them zero
        workspace = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
    _dev(out, workspace)
    lw = _LayerWeights(*[t.data_ptr() for t in ws])
    _check(entry(dtype_code(x.dtype), ctypes.byref(lw), _ptr(x), _ptr(local_mask),
                 _ptr(global_mask), B, S, D, H, F, W, G, attn_scale, ln_eps, _ptr(out),
                 _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev)))
    return out


def encoder_forward_workspace_bytes(dtype, B, S, hidden, H, ffn, W, G) -> int:
    return int(load_library().lf_encoder_forward_workspace_bytes(dtype_code(dtype), B, S, hidden,
                                                                 H, ffn, W, G))


def encoder_forward(x, layers: list, local_mask, global_mask, H: int, W: int, G: int,
                    attn_scale: float = 0.125, ln_eps: float = 1e-5, out=None, workspace=None,
                    any_globals: bool = False):
    """[FT-LF computation flow] preprocessing once, then len(layers) encoder layers -> y.

    any_globals: the global tokens may sit at any positions (lf_encoder_forward_any_globals).
    """
    lib = load_library()
    entry = lib.lf_encoder_forward_any_globals if any_globals else lib.lf_encoder_forward
    if not layers:
        raise ValueError("at least one layer")
    ws = [[lw[n] for n in LAYER_WEIGHT_FIELDS] for lw in layers]
    dev = _dev(x, local_mask, global_mask, *[t for w in ws for t in w])
    B, S, D = x.shape
    F = layers[0]["w_ffn1"].shape[0]
    if out is None:
        out = torch.empty_like(x)
    nbytes = encoder_forward_workspace_bytes(x.dtype, B, S, D, H, F, W, G)
    if workspace is None:
        # the leading split tickets must start at zero; the library leaves them zero
        workspace = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
    _dev(out, workspace)
    arr = (_LayerWeights * len(layers))(*[_LayerWeights(*[t.data_ptr() for t in w]) for w in ws])
    _check(entry(dtype_code(x.dtype), arr, len(layers), _ptr(x), _ptr(local_mask),
                 _ptr(global_mask), B, S, D, H, F, W, G, attn_scale, ln_eps, _ptr(out),
                 _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev)))
    return out


def ffn_block_workspace_bytes(dtype, M, D, F, fused: bool) -> int:
    return int(load_library().lf_ffn_block_workspace_bytes(dtype_code(dtype), M, D, F,
                                                           1 if fused else 0))


def ffn_block(h, resid, w1, b1, w2, b2, ln_g, ln_b, fused: bool, ln_eps: float = 1e-5,
              out=None, workspace=None):
    """[FT-LF computation flow, per-layer step 6] y = LN(resid + GELU(h W1^T + b1) W2^T + b2).

    h [M, D] (fp16 / bf16 / fp32), resid [M, D] fp32; fused selects the one-kernel
    path (the intermediate stays on chip) over the two GEMMs the layer runs.
    """
    lib = load_library()
    dev = _dev(h, resid, w1, b1, w2, b2, ln_g, ln_b)
    if resid.dtype != torch.float32:
        raise TypeError("resid must be float32 (the residual stream)")
    M, D = h.shape
    F = w1.shape[0]
    if out is None:
        out = torch.empty_like(h)
    nbytes = ffn_block_workspace_bytes(h.dtype, M, D, F, fused)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    _dev(out, workspace)
    _check(lib.lf_ffn_block(dtype_code(h.dtype), _ptr(h), _ptr(resid), _ptr(w1), _ptr(b1),
                            _ptr(w2), _ptr(b2), _ptr(ln_g), _ptr(ln_b), M, D, F, ln_eps,
                            1 if fused else 0, _ptr(out), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(dev)))
    return out
