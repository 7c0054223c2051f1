"""MI355X (gfx950) hybrid attention core of ZGCM-1: Python binding of the C ABI in include/zg_attn.h.

The binding only marshals arguments: it checks dtypes/devices/shapes, takes raw device pointers and
the current HIP stream from torch, and calls libzgattn.so through ctypes. Every step of the path runs
in the library's kernels; there is no fallback. If the library is missing the call raises.

Build the library with ``python -m global_causal_attention_amd.build`` (hipcc, --offload-arch=gfx950).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

from ._abi import (LIB_PATH, ZgAttnCfg, ZgTokenStrides, load_library, ZG_OK, ZG_ERR_NULL,
                   ZG_ERR_SHAPE, ZG_ERR_UNSUPPORTED, ZG_ERR_WORKSPACE, ZG_ERR_HIP, EXPORTS)

__all__ = ["AttnConfig", "ZGError", "zg_attn_prefill", "zg_attn_prefill_cached",
           "zg_attn_forward_train", "zg_attn_forward_train_workspace_bytes", "zg_attn_backward",
           "zg_attn_backward_workspace_bytes",
           "zg_hbm_read_probe", "zg_attn_decode", "zg_attn_decode_noalloc", "zg_attn_decode_fp8",
           "zg_kv_to_fp8", "zg_kv_bytes",
           "zg_attn_prefill_workspace_bytes", "zg_attn_decode_workspace_bytes", "zg_rmsnorm",
           "zg_gemm_bf16", "zg_attn_layer", "zg_attn_layer_workspace_bytes", "zg_rmsnorm_fp8",
           "zg_quant_rows_fp8", "zg_gemm_fp8", "zg_attn_layer_fp8",
           "zg_attn_layer_fp8_workspace_bytes", "zg_last_error", "load_library", "LIB_PATH",
           "EXPORTS"]


class ZGError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"zg status {status}: {msg}")
        self.status = status


@dataclass(frozen=True)
class AttnConfig:
    """One attention layer. Defaults are ZGCM-1's local layer (zh-TW translation page, section 2.1):
    32 query / 8 KV heads of dim 128, window 128, gated, partial RoPE on floor(0.33*128) = 42 dims."""
    n_q_heads: int = 32
    n_kv_heads: int = 8
    head_dim: int = 128
    window: int = 128
    gated: bool = True
    rot_dim: int = 42
    rope_base: float = 1e4
    rms_eps: float = 1e-6
    softmax_scale: float = 0.0

    def c(self) -> ZgAttnCfg:
        return ZgAttnCfg(self.n_q_heads, self.n_kv_heads, self.head_dim, self.window,
                         1 if self.gated else 0, self.rot_dim, float(self.rope_base),
                         float(self.rms_eps), float(self.softmax_scale))


def _check(status: int):
    if status != ZG_OK:
        raise ZGError(status, zg_last_error())


def zg_last_error() -> str:
    return load_library().zg_last_error().decode()


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, device_required=True):
    import torch
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device_required and not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def _token_stride(t, name, row):
    """Element stride between tokens of a [B, T, H, D] (or [B*T, row]) view whose rows are dense."""
    if t.dim() == 4:
        if t.stride(3) != 1 or t.stride(2) != t.shape[3]:
            raise ValueError(f"{name}: heads and dims must be dense")
        st = t.stride(1)
        if t.shape[0] > 1 and t.stride(0) != st * t.shape[1]:
            raise ValueError(f"{name}: batch stride must equal T * token stride")
        return st
    raise ValueError(f"{name} must be 4-D [B, T, H, D]")


def _shape(t, name, shape):
    """Raise ValueError unless tensor t has exactly `shape` (checked before any launch: the
    library addresses caches and rows from cfg and the sizes it is given, not from the tensors)."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}; expected {tuple(shape)}")


def _norm_weights(q_norm_w, k_norm_w, head_dim):
    import torch
    for w, n in ((q_norm_w, "q_norm_w"), (k_norm_w, "k_norm_w")):
        if w is not None:
            _shape(w, n, (head_dim,))
            _need(w, n, torch.float32)
            if not w.is_contiguous():
                raise ValueError(f"{n} must be contiguous")


def _layer_shapes(cfg, q, k, v, gate):
    """[B, T, Hq, D] q (and gate), [B, T, Hkv, D] k and v, against cfg; returns (B, T)."""
    if q.dim() != 4:
        raise ValueError(f"q must be 4-D [B, T, Hq, D], got shape {tuple(q.shape)}")
    B, T = q.shape[:2]
    _shape(q, "q", (B, T, cfg.n_q_heads, cfg.head_dim))
    _shape(k, "k", (B, T, cfg.n_kv_heads, cfg.head_dim))
    _shape(v, "v", (B, T, cfg.n_kv_heads, cfg.head_dim))
    if cfg.gated:
        if gate is None:
            raise ValueError("gate is required when cfg.gated")
        _shape(gate, "gate", (B, T, cfg.n_q_heads, cfg.head_dim))
    return B, T


def _decode_shapes(cfg, q_new, k_new, v_new, gate, k_cache, v_cache, seqlens, max_seqlen):
    """One new token per sequence: q_new/gate [B, Hq, D], k_new/v_new [B, Hkv, D]; ring caches
    [B, W, Hkv, D] (the library writes slot pos % W), linear caches [B, rows, Hkv, D] with
    rows >= max_seqlen; seqlens [B]."""
    if q_new.dim() != 3:
        raise ValueError(f"q_new must be 3-D [B, Hq, D], got shape {tuple(q_new.shape)}")
    B = q_new.shape[0]
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    _shape(q_new, "q_new", (B, Hq, D))
    _shape(k_new, "k_new", (B, Hkv, D))
    _shape(v_new, "v_new", (B, Hkv, D))
    if cfg.gated:
        if gate is None:
            raise ValueError("gate is required when cfg.gated")
        _shape(gate, "gate", (B, Hq, D))
    rows = cfg.window if cfg.window > 0 else k_cache.shape[1]
    _shape(k_cache, "k_cache", (B, rows, Hkv, D))
    _shape(v_cache, "v_cache", (B, rows, Hkv, D))
    if cfg.window == 0 and rows < max_seqlen:
        raise ValueError(f"linear caches hold {rows} rows < max_seqlen={max_seqlen}")
    if seqlens.dim() != 1 or seqlens.numel() != B:
        raise ValueError(f"seqlens must hold one length per sequence ({B}), got shape "
                         f"{tuple(seqlens.shape)}")
    return B


def zg_attn_prefill_workspace_bytes(cfg: AttnConfig, B: int, T: int) -> int:
    c = cfg.c()
    return load_library().zg_attn_prefill_workspace_bytes(ctypes.byref(c), B, T)


def zg_attn_prefill(cfg: AttnConfig, q, k, v, gate=None, *, q_norm_w=None, k_norm_w=None,
                    pos0: int = 0, out=None, workspace=None, stream=None):
    """Prefill attention (see include/zg_attn.h). q, gate: [B, T, Hq, 128] bf16; k, v:
    [B, T, Hkv, 128] bf16 (token-strided views allowed). Returns out [B, T, Hq, 128] bf16."""
    import torch
    bf = torch.bfloat16
    B, T = _layer_shapes(cfg, q, k, v, gate)
    Hq, D = cfg.n_q_heads, cfg.head_dim
    _shape(out, "out", (B, T, Hq, D))
    _norm_weights(q_norm_w, k_norm_w, D)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, bf)
    if cfg.gated:
        _need(gate, "gate", bf)
    if out is None:
        out = torch.empty((B, T, Hq, D), dtype=bf, device=q.device)
    _need(out, "out", bf)
    strides = ZgTokenStrides(_token_stride(q, "q", Hq * D), _token_stride(k, "k", 0),
                             _token_stride(v, "v", 0),
                             _token_stride(gate, "gate", 0) if cfg.gated else Hq * D,
                             _token_stride(out, "out", 0))
    need = zg_attn_prefill_workspace_bytes(cfg, B, T)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    c = cfg.c()
    _check(load_library().zg_attn_prefill(
        ctypes.byref(c), B, T, pos0, _ptr(q), _ptr(k), _ptr(v), _ptr(gate if cfg.gated else None),
        _ptr(q_norm_w), _ptr(k_norm_w), ctypes.byref(strides), _ptr(out), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def _packed(t, name, shape):
    if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor of shape {tuple(shape)}")


def zg_attn_forward_train_workspace_bytes(cfg: AttnConfig, B: int, T: int) -> int:
    c = cfg.c()
    return load_library().zg_attn_forward_train_workspace_bytes(ctypes.byref(c), B, T)


def zg_attn_forward_train(cfg: AttnConfig, q, k, v, gate=None, *, out=None, lse=None,
                          workspace=None, stream=None):
    """Forward for training (see include/zg_attn.h): packed q, gate [B, T, Hq, 128] and k, v
    [B, T, Hkv, 128] bf16, positions 0 .. T-1, norm weights 1. Returns (out, lse) with lse the
    [B, T, Hq] fp32 natural-log log-sum-exp of each query row's scaled scores."""
    import torch
    bf = torch.bfloat16
    B, T = _layer_shapes(cfg, q, k, v, gate)
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    _shape(out, "out", (B, T, Hq, D))
    _shape(lse, "lse", (B, T, Hq))
    for t, n, shp in ((q, "q", (B, T, Hq, D)), (k, "k", (B, T, Hkv, D)), (v, "v", (B, T, Hkv, D))):
        _need(t, n, bf)
        _packed(t, n, shp)
    if cfg.gated:
        _need(gate, "gate", bf)
        _packed(gate, "gate", (B, T, Hq, D))
    if out is None:
        out = torch.empty((B, T, Hq, D), dtype=bf, device=q.device)
    if lse is None:
        lse = torch.empty((B, T, Hq), dtype=torch.float32, device=q.device)
    _need(out, "out", bf)
    _packed(out, "out", (B, T, Hq, D))
    _need(lse, "lse", torch.float32)
    _packed(lse, "lse", (B, T, Hq))
    need = zg_attn_forward_train_workspace_bytes(cfg, B, T)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    c = cfg.c()
    _check(load_library().zg_attn_forward_train(
        ctypes.byref(c), B, T, _ptr(q), _ptr(k), _ptr(v), _ptr(gate if cfg.gated else None),
        _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out, lse


def zg_attn_backward_workspace_bytes(cfg: AttnConfig, B: int, T: int) -> int:
    c = cfg.c()
    return load_library().zg_attn_backward_workspace_bytes(ctypes.byref(c), B, T)


def zg_attn_backward(cfg: AttnConfig, q, k, v, gate, out, dout, lse, *, workspace=None,
                     stream=None):
    """Backward pass (see include/zg_attn.h) from the forward's inputs, its out and lse and the
    output gradient dout. Returns (dq, dk, dv, dgate); dgate is None when not gated."""
    import torch
    bf = torch.bfloat16
    B, T = _layer_shapes(cfg, q, k, v, gate)
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    _shape(out, "out", (B, T, Hq, D))
    _shape(dout, "dout", (B, T, Hq, D))
    _shape(lse, "lse", (B, T, Hq))
    for t, n, shp in ((q, "q", (B, T, Hq, D)), (k, "k", (B, T, Hkv, D)), (v, "v", (B, T, Hkv, D)),
                      (out, "out", (B, T, Hq, D)), (dout, "dout", (B, T, Hq, D))):
        _need(t, n, bf)
        _packed(t, n, shp)
    if cfg.gated:
        _need(gate, "gate", bf)
        _packed(gate, "gate", (B, T, Hq, D))
    _need(lse, "lse", torch.float32)
    _packed(lse, "lse", (B, T, Hq))
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dgate = torch.empty_like(q) if cfg.gated else None
    need = zg_attn_backward_workspace_bytes(cfg, B, T)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    c = cfg.c()
    _check(load_library().zg_attn_backward(
        ctypes.byref(c), B, T, _ptr(q), _ptr(k), _ptr(v), _ptr(gate if cfg.gated else None),
        _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dgate),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return dq, dk, dv, dgate


def zg_attn_prefill_cached_workspace_bytes(cfg: AttnConfig, B: int, T: int) -> int:
    c = cfg.c()
    return load_library().zg_attn_prefill_cached_workspace_bytes(ctypes.byref(c), B, T)


def zg_attn_prefill_cached(cfg: AttnConfig, q, k, v, gate, k_cache, v_cache, *, pos0: int,
                           q_norm_w=None, k_norm_w=None, out=None, workspace=None, stream=None):
    """Chunked prefill through the decode caches (see include/zg_attn.h): the T new tokens sit at
    positions pos0 .. pos0+T-1; k_cache/v_cache are [B, W, Hkv, 128] rings (window > 0) or
    [B, stride, Hkv, 128] linear caches (window 0), read for earlier positions and updated with
    the new tokens. Returns out [B, T, Hq, 128] bf16."""
    import torch
    bf = torch.bfloat16
    B, T = _layer_shapes(cfg, q, k, v, gate)
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    _shape(out, "out", (B, T, Hq, D))
    rows = cfg.window if cfg.window > 0 else k_cache.shape[1]
    _shape(k_cache, "k_cache", (B, rows, Hkv, D))
    _shape(v_cache, "v_cache", (B, rows, Hkv, D))
    if cfg.window == 0 and rows < pos0 + T:
        raise ValueError(f"linear caches hold {rows} rows < pos0 + T = {pos0 + T}")
    _norm_weights(q_norm_w, k_norm_w, D)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, bf)
    if cfg.gated:
        _need(gate, "gate", bf)
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, n, bf)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    if out is None:
        out = torch.empty((B, T, Hq, D), dtype=bf, device=q.device)
    _need(out, "out", bf)
    strides = ZgTokenStrides(_token_stride(q, "q", Hq * D), _token_stride(k, "k", 0),
                             _token_stride(v, "v", 0),
                             _token_stride(gate, "gate", 0) if cfg.gated else Hq * D,
                             _token_stride(out, "out", 0))
    need = zg_attn_prefill_cached_workspace_bytes(cfg, B, T)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    c = cfg.c()
    _check(load_library().zg_attn_prefill_cached(
        ctypes.byref(c), B, T, pos0, _ptr(q), _ptr(k), _ptr(v), _ptr(gate if cfg.gated else None),
        _ptr(q_norm_w), _ptr(k_norm_w), ctypes.byref(strides), _ptr(k_cache), _ptr(v_cache),
        k_cache.shape[1], _ptr(out), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def zg_attn_decode_workspace_bytes(cfg: AttnConfig, B: int, max_seqlen: int) -> int:
    c = cfg.c()
    return load_library().zg_attn_decode_workspace_bytes(ctypes.byref(c), B, max_seqlen)


def zg_attn_decode(cfg: AttnConfig, q_new, k_new, v_new, gate, k_cache, v_cache, seqlens, *,
                   max_seqlen: int, q_norm_w=None, k_norm_w=None, out=None, workspace=None,
                   stream=None):
    """One decode step (see include/zg_attn.h). Updates k_cache / v_cache in place and returns
    out [B, Hq, 128] bf16."""
    import torch
    bf = torch.bfloat16
    B = _decode_shapes(cfg, q_new, k_new, v_new, gate, k_cache, v_cache, seqlens, max_seqlen)
    _shape(out, "out", q_new.shape)
    for t, n in ((q_new, "q_new"), (k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"),
                 (v_cache, "v_cache")):
        _need(t, n, bf)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    _need(seqlens, "seqlens", torch.int32)
    if cfg.gated:
        _need(gate, "gate", bf)
        if not gate.is_contiguous():
            raise ValueError("gate must be contiguous")
    _norm_weights(q_norm_w, k_norm_w, cfg.head_dim)
    if out is None:
        out = torch.empty_like(q_new)
    _need(out, "out", bf)
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    need = zg_attn_decode_workspace_bytes(cfg, B, max_seqlen)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_new.device)
    stride = k_cache.shape[1]
    c = cfg.c()
    _check(load_library().zg_attn_decode(
        ctypes.byref(c), B, stride, max_seqlen, _ptr(q_new), _ptr(k_new), _ptr(v_new),
        _ptr(gate if cfg.gated else None), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(k_cache),
        _ptr(v_cache), _ptr(seqlens), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def zg_attn_decode_noalloc(cfg: AttnConfig, q_new, k_new, v_new, gate, k_cache, v_cache, seqlens,
                           *, max_seqlen: int, q_norm_w=None, k_norm_w=None, out=None,
                           stream=None):
    """zg_attn_decode with the library's static per-device scratch instead of a workspace (see
    include/zg_attn.h): the library call allocates nothing (`out` is allocated here when not
    given). Calls that overlap on one GPU race on the shared scratch."""
    import torch
    bf = torch.bfloat16
    _decode_shapes(cfg, q_new, k_new, v_new, gate, k_cache, v_cache, seqlens, max_seqlen)
    _shape(out, "out", q_new.shape)
    for t, n in ((q_new, "q_new"), (k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"),
                 (v_cache, "v_cache")):
        _need(t, n, bf)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    _need(seqlens, "seqlens", torch.int32)
    if cfg.gated:
        _need(gate, "gate", bf)
        if not gate.is_contiguous():
            raise ValueError("gate must be contiguous")
    _norm_weights(q_norm_w, k_norm_w, cfg.head_dim)
    if out is None:
        out = torch.empty_like(q_new)
    _need(out, "out", bf)
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    c = cfg.c()
    _check(load_library().zg_attn_decode_noalloc(
        ctypes.byref(c), q_new.shape[0], k_cache.shape[1], max_seqlen, _ptr(q_new), _ptr(k_new),
        _ptr(v_new), _ptr(gate if cfg.gated else None), _ptr(q_norm_w), _ptr(k_norm_w),
        _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(out), _stream(stream)))
    return out


def zg_attn_decode_fp8(cfg: AttnConfig, q_new, k_new, v_new, gate, k_cache, v_cache, seqlens, *,
                       max_seqlen: int, k_scale: float = 1.0, v_scale: float = 1.0, q_norm_w=None,
                       k_norm_w=None, out=None, workspace=None, stream=None):
    """One decode step over E4M3 caches (torch.float8_e4m3fn or uint8 tensors of the bf16 cache
    shape; see include/zg_attn.h). Updates the caches in place, returns out [B, Hq, 128] bf16."""
    import torch
    bf = torch.bfloat16
    B = _decode_shapes(cfg, q_new, k_new, v_new, gate, k_cache, v_cache, seqlens, max_seqlen)
    _shape(out, "out", q_new.shape)
    for t, n in ((q_new, "q_new"), (k_new, "k_new"), (v_new, "v_new")):
        _need(t, n, bf)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        if t.dtype not in (torch.float8_e4m3fn, torch.uint8) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous float8_e4m3fn or uint8 device tensor")
    _need(seqlens, "seqlens", torch.int32)
    if cfg.gated:
        _need(gate, "gate", bf)
        if not gate.is_contiguous():
            raise ValueError("gate must be contiguous")
    _norm_weights(q_norm_w, k_norm_w, cfg.head_dim)
    if out is None:
        out = torch.empty_like(q_new)
    _need(out, "out", bf)
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    need = zg_attn_decode_workspace_bytes(cfg, B, max_seqlen)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_new.device)
    c = cfg.c()
    _check(load_library().zg_attn_decode_fp8(
        ctypes.byref(c), B, k_cache.shape[1], max_seqlen, _ptr(q_new), _ptr(k_new), _ptr(v_new),
        _ptr(gate if cfg.gated else None), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(k_cache),
        _ptr(v_cache), float(k_scale), float(v_scale), _ptr(seqlens), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def zg_kv_to_fp8(src, scale: float = 1.0, out=None, stream=None):
    """E4M3 copy of a bf16 device tensor (values / scale, nearest-even, saturating at +-448)."""
    import torch
    _need(src, "src", torch.bfloat16)
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    if out is None:
        out = torch.empty(src.shape, dtype=torch.float8_e4m3fn, device=src.device)
    _check(load_library().zg_kv_to_fp8(_ptr(src), _ptr(out), src.numel(), float(scale),
                                       _stream(stream)))
    return out


def zg_kv_bytes(n_layers, global_every, n_kv_heads, head_dim, window, elem_bytes, batch,
                seqlen) -> int:
    """KV-cache bytes of a layer stack (pure host arithmetic in the library)."""
    lib = load_library()
    r = lib.zg_kv_bytes(n_layers, global_every, n_kv_heads, head_dim, window, elem_bytes, batch,
                        seqlen)
    if r == 0 and min(n_layers, global_every, n_kv_heads, head_dim, window, elem_bytes, batch,
                      seqlen) < 0:
        raise ZGError(ZG_ERR_SHAPE, zg_last_error())
    return r


def zg_hbm_read_probe(src, sink=None, n_blocks=2048, stream=None):
    """Streaming-read probe over the bytes of the device tensor `src` (see include/zg_attn.h);
    returns the sink tensor (one meaningless word per wave)."""
    import torch
    nbytes = src.numel() * src.element_size()
    if sink is None:
        sink = torch.empty(4 * n_blocks, dtype=torch.int32, device=src.device)
    _check(load_library().zg_hbm_read_probe(_ptr(src), nbytes - nbytes % 16, _ptr(sink), n_blocks,
                                            _stream(stream)))
    return sink


def zg_rmsnorm(x, eps=1e-6, w=None, out=None, stream=None):
    import torch
    _shape(w, "w", (x.shape[-1],))
    _shape(out, "out", x.shape)
    _need(x, "x", torch.float32)
    if not x.is_contiguous() or (w is not None and not w.is_contiguous()):
        raise ValueError("x and w must be contiguous")
    if w is not None:
        _need(w, "w", torch.float32)
    rows = x.numel() // x.shape[-1]
    if out is None:
        out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    _check(load_library().zg_rmsnorm(rows, x.shape[-1], _ptr(x), _ptr(w), float(eps), _ptr(out),
                                     _stream(stream)))
    return out


def zg_gemm_bf16(x, w, residual=None, y=None, want_y=True, stream=None):
    """Y = X W^T (fp32 accumulate); residual (fp32) += Y if given; y = bf16(Y) if want_y."""
    import torch
    if x.dim() != 2 or w.dim() != 2:
        raise ValueError(f"x [M, K] and w [N, K] must be 2-D, got {tuple(x.shape)} and {tuple(w.shape)}")
    M, K = x.shape
    N = w.shape[0]
    _shape(w, "w", (N, K))
    _shape(residual, "residual", (M, N))
    _shape(y, "y", (M, N))
    _need(x, "x", torch.bfloat16)
    _need(w, "w", torch.bfloat16)
    for t, n in ((x, "x"), (w, "w"), (residual, "residual"), (y, "y")):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    if residual is not None:
        _need(residual, "residual", torch.float32)
    if want_y and y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check(load_library().zg_gemm_bf16(M, N, K, _ptr(x), _ptr(w), _ptr(residual),
                                       _ptr(y if want_y else None), N, _stream(stream)))
    return y if want_y else residual


def zg_attn_layer_workspace_bytes(cfg: AttnConfig, B: int, T: int) -> int:
    c = cfg.c()
    return load_library().zg_attn_layer_workspace_bytes(ctypes.byref(c), B, T)


def zg_attn_layer(cfg: AttnConfig, x, w_qkvg, w_o, *, q_norm_w=None, k_norm_w=None,
                  workspace=None, stream=None):
    """x (fp32 [B, T, hidden]) <- x + o_proj(attn(RMSNorm(x))), in place."""
    import torch
    if x.dim() != 3:
        raise ValueError(f"x must be 3-D [B, T, hidden], got shape {tuple(x.shape)}")
    B, T, hidden = x.shape
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    _shape(x, "x", (B, T, Hq * D))
    _shape(w_qkvg, "w_qkvg", ((Hq + 2 * Hkv + (Hq if cfg.gated else 0)) * D, hidden))
    _shape(w_o, "w_o", (hidden, Hq * D))
    _need(x, "x", torch.float32)
    _need(w_qkvg, "w_qkvg", torch.bfloat16)
    _need(w_o, "w_o", torch.bfloat16)
    for t, n in ((x, "x"), (w_qkvg, "w_qkvg"), (w_o, "w_o")):
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    _norm_weights(q_norm_w, k_norm_w, D)
    need = zg_attn_layer_workspace_bytes(cfg, B, T)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    c = cfg.c()
    _check(load_library().zg_attn_layer(
        ctypes.byref(c), B, T, _ptr(x), _ptr(w_qkvg), _ptr(w_o), _ptr(q_norm_w), _ptr(k_norm_w),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return x


# ---- E4M3 projections: codes as torch.uint8, one fp32 scale per row ----

def zg_rmsnorm_fp8(x, eps=1e-6, w=None, out=None, scale=None, stream=None):
    """E4M3 rows of RMSNorm(x) * w (x fp32 [..., dim]): returns (codes uint8 [..., dim],
    scale fp32 [rows]); row r stands for decode(codes[r]) * scale[r]."""
    import torch
    dim = x.shape[-1]
    rows = x.numel() // dim
    _shape(w, "w", (dim,))
    _shape(out, "out", x.shape)
    _shape(scale, "scale", (rows,))
    _need(x, "x", torch.float32)
    if not x.is_contiguous() or (w is not None and not w.is_contiguous()):
        raise ValueError("x and w must be contiguous")
    if w is not None:
        _need(w, "w", torch.float32)
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(rows, dtype=torch.float32, device=x.device)
    _need(out, "out", torch.uint8)
    _need(scale, "scale", torch.float32)
    _check(load_library().zg_rmsnorm_fp8(rows, dim, _ptr(x), _ptr(w), float(eps), _ptr(out),
                                         _ptr(scale), _stream(stream)))
    return out, scale


def zg_quant_rows_fp8(x, out=None, scale=None, stream=None):
    """E4M3 rows of the bf16 matrix x [rows, dim] (rows may be strided, elements dense): returns
    (codes uint8 [rows, dim], scale fp32 [rows])."""
    import torch
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError(f"x must be a 2-D [rows, dim] view with dense rows, got shape {tuple(x.shape)}")
    rows, dim = x.shape
    _shape(out, "out", (rows, dim))
    _shape(scale, "scale", (rows,))
    _need(x, "x", torch.bfloat16)
    if out is None:
        out = torch.empty((rows, dim), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(rows, dtype=torch.float32, device=x.device)
    _need(out, "out", torch.uint8)
    _need(scale, "scale", torch.float32)
    _check(load_library().zg_quant_rows_fp8(rows, dim, _ptr(x), x.stride(0), _ptr(out), _ptr(scale),
                                            _stream(stream)))
    return out, scale


def zg_gemm_fp8(x, x_scale, w, w_scale, residual=None, y=None, want_y=True, stream=None):
    """Y = diag(x_scale) X W^T diag(w_scale) for E4M3 codes X [M, K], W [N, K] (fp32 accumulate);
    residual (fp32) += Y if given; y = bf16(Y) if want_y."""
    import torch
    if x.dim() != 2 or w.dim() != 2:
        raise ValueError(f"x [M, K] and w [N, K] must be 2-D, got {tuple(x.shape)} and {tuple(w.shape)}")
    M, K = x.shape
    N = w.shape[0]
    _shape(w, "w", (N, K))
    _shape(x_scale, "x_scale", (M,))
    _shape(w_scale, "w_scale", (N,))
    _shape(residual, "residual", (M, N))
    _shape(y, "y", (M, N))
    _need(x, "x", torch.uint8)
    _need(w, "w", torch.uint8)
    _need(x_scale, "x_scale", torch.float32)
    _need(w_scale, "w_scale", torch.float32)
    for t, n in ((x, "x"), (w, "w"), (x_scale, "x_scale"), (w_scale, "w_scale"),
                 (residual, "residual"), (y, "y")):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    if residual is not None:
        _need(residual, "residual", torch.float32)
    if want_y and y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check(load_library().zg_gemm_fp8(M, N, K, _ptr(x), _ptr(x_scale), _ptr(w), _ptr(w_scale),
                                      _ptr(residual), _ptr(y if want_y else None), N,
                                      _stream(stream)))
    return y if want_y else residual


def zg_attn_layer_fp8_workspace_bytes(cfg: AttnConfig, B: int, T: int) -> int:
    c = cfg.c()
    return load_library().zg_attn_layer_fp8_workspace_bytes(ctypes.byref(c), B, T)


def zg_attn_layer_fp8(cfg: AttnConfig, x, w_qkvg, s_qkvg, w_o, s_o, *, q_norm_w=None,
                      k_norm_w=None, workspace=None, stream=None):
    """zg_attn_layer with E4M3 projections (weights as codes + per-row scales, e.g. from
    zg_quant_rows_fp8 of the bf16 weights); x (fp32 [B, T, hidden]) is updated in place."""
    import torch
    if x.dim() != 3:
        raise ValueError(f"x must be 3-D [B, T, hidden], got shape {tuple(x.shape)}")
    B, T, hidden = x.shape
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    n_qkvg = (Hq + 2 * Hkv + (Hq if cfg.gated else 0)) * D
    _shape(x, "x", (B, T, Hq * D))
    _shape(w_qkvg, "w_qkvg", (n_qkvg, hidden))
    _shape(s_qkvg, "s_qkvg", (n_qkvg,))
    _shape(w_o, "w_o", (hidden, Hq * D))
    _shape(s_o, "s_o", (hidden,))
    _need(x, "x", torch.float32)
    _need(w_qkvg, "w_qkvg", torch.uint8)
    _need(w_o, "w_o", torch.uint8)
    _need(s_qkvg, "s_qkvg", torch.float32)
    _need(s_o, "s_o", torch.float32)
    for t, n in ((x, "x"), (w_qkvg, "w_qkvg"), (w_o, "w_o"), (s_qkvg, "s_qkvg"), (s_o, "s_o")):
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    _norm_weights(q_norm_w, k_norm_w, D)
    need = zg_attn_layer_fp8_workspace_bytes(cfg, B, T)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    c = cfg.c()
    _check(load_library().zg_attn_layer_fp8(
        ctypes.byref(c), B, T, _ptr(x), _ptr(w_qkvg), _ptr(s_qkvg), _ptr(w_o), _ptr(s_o),
        _ptr(q_norm_w), _ptr(k_norm_w), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return x
