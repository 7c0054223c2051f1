"""Test-side rounding model of the attention stack as the GPU library evaluates it.

The fp64 oracle (oracle/stack.py) rounds nothing. The GPU rounds to bf16 at fixed points, and over
32 residual layers those roundings move the output by more than the bf16 output bar. This model is
the oracle's arithmetic in fp64 with a bf16 rounding (round to nearest even) inserted exactly where
the library rounds, so that a comparison with it separates the rounding the design asks for from a
wiring mistake. It is built on the oracle's own prologue (RMSNorm then partial RoPE) and shares
nothing with the GPU code.

Rounding points (ZGCM-1 zh-TW translation page, section 2.1 and Fig. 3 for the layer; section 3.1
for Pre-LN):
  * h = bf16(RMSNorm(x)) (the residual x itself is fp32 and is not rounded);
  * the q, k, v and gate projections h W^T, each rounded to bf16;
  * global layers (full causal, ungated), and local layers whose window covers the whole sequence
    (T <= 128: the library runs them as causal, gated): the matrix cores see bf16(q_hat * c) and
    bf16(k_hat), c = log2(e) / sqrt(128); scores are in log2 units and the softmax weights are
    bf16(exp2(s)) (with weight-1 norms |s| <= 128 c < 32, so the running reference of the causal
    kernel stays 0);
  * local layers with T > 128 (window 128, gated, 4 query heads per KV head, 42 rotary dims,
    the banded kernel): the matrix cores see
    q with its first 42 dims replaced by bf16(RoPE(q)) and bf16(k_hat * c); the RMS factor r_q of
    the query multiplies the scores; the weights are bf16(exp2(r_q (s - mu))) with mu the bf16
    rounding of the largest score of the first 32-key block the banded kernel visits for that query
    (keys 64 tc - 32 .. 64 tc - 1 for a query in the 64-query step tc >= 1, keys 0 .. 31 in step 0);
  * the normaliser sums the rounded weights; the attention output (times sigmoid(g) on local
    layers) is rounded to bf16 before o_proj; o_proj adds h_attn W_o^T to the residual.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

C_LOG2 = np.log2(np.e) / np.sqrt(128.0)


def bf16(x):
    """Round to nearest-even bfloat16 (through float32, as the GPU rounds its fp32 values),
    returned as float64."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def _rms_rows(x, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def _first_block(t):
    """Key range [lo, hi) of the first 32-key block the banded kernel visits for query row t."""
    tc = t // 64
    return (64 * tc - 32, 64 * tc) if tc >= 1 else (0, 32)


def attention_causal(q, k, v, rope_base, g=None, eps=1e-6):
    """q: [T, 32, 128] (bf16 values), k, v: [T, 8, 128]; full causal; gated when g is given (a
    local layer whose window covers the whole sequence runs this form)."""
    T = q.shape[0]
    pos = np.arange(T)
    qs = bf16(C_LOG2 * oracle.qk_prologue(q, pos, None, rot_dim=42, rope_base=rope_base, eps=eps))
    ks = bf16(oracle.qk_prologue(k, pos, None, rot_dim=42, rope_base=rope_base, eps=eps))
    out = np.empty(q.shape)
    for h in range(32):
        c = h // 4
        s = qs[:, h] @ ks[:, c].T                                   # [T, T], log2 units
        s = np.where(np.tril(np.ones((T, T), dtype=bool)), s, -np.inf)
        p = bf16(np.exp2(s))
        out[:, h] = (p @ v[:, c]) / p.sum(-1, keepdims=True)
    if g is not None:
        out = out / (1.0 + np.exp(-g))
    return bf16(out)


def attention_local(q, k, v, g, rope_base, window=128, eps=1e-6):
    """q, g: [T, 32, 128] (bf16 values), k, v: [T, 8, 128]; banded, gated."""
    T = q.shape[0]
    pos = np.arange(T)
    r_q = 1.0 / np.sqrt(np.mean(q * q, axis=-1) + eps)                     # [T, 32]
    qf = q.copy()
    qf[..., :42] = bf16(oracle.partial_rope(q, pos, 42, rope_base)[..., :42])
    ks = bf16(C_LOG2 * oracle.qk_prologue(k, pos, None, rot_dim=42, rope_base=rope_base, eps=eps))
    out = np.empty(q.shape)
    for t in range(T):
        lo = max(0, t - window + 1)
        f0, f1 = _first_block(t)
        f0, f1 = max(f0, lo), min(f1, t + 1)
        for c in range(8):
            s = qf[t, 4 * c:4 * c + 4] @ ks[lo:t + 1, c].T                   # [4, n] raw scores
            mu = bf16(s[:, f0 - lo:f1 - lo].max(-1, keepdims=True))
            p = bf16(np.exp2(r_q[t, 4 * c:4 * c + 4, None] * (s - mu)))
            o = (p @ v[lo:t + 1, c]) / p.sum(-1, keepdims=True)
            out[t, 4 * c:4 * c + 4] = o / (1.0 + np.exp(-g[t, 4 * c:4 * c + 4]))
    return bf16(out)


def layer(x, w, *, is_global, rope_base=1e7, window=128, eps=1e-6):
    """One Pre-LN layer on one sequence. x: [T, 4096] float64 residual; w: dict of [out, in]
    float64 weights (bf16 values) 'wq', 'wk', 'wv', 'wo' and, for local layers, 'wg'."""
    T = x.shape[0]
    h = bf16(_rms_rows(x, eps))
    q = bf16(h @ w["wq"].T).reshape(T, 32, 128)
    k = bf16(h @ w["wk"].T).reshape(T, 8, 128)
    v = bf16(h @ w["wv"].T).reshape(T, 8, 128)
    if is_global:
        a = attention_causal(q, k, v, rope_base, eps=eps)
    else:
        g = bf16(h @ w["wg"].T).reshape(T, 32, 128)
        if T <= window:   # the window covers every key: the causal form, gated
            a = attention_causal(q, k, v, rope_base, g=g, eps=eps)
        else:
            a = attention_local(q, k, v, g, rope_base, window=window, eps=eps)
    return x + a.reshape(T, 4096) @ w["wo"].T

