"""fp64 oracle of the attention-only 32-layer stack with projections. TEST INFRASTRUCTURE ONLY.

ZGCM-1 zh-TW translation page §2.1 and Fig. 3: a normalised hidden state h feeds parallel q, k, v and
gate projections; q and k get RMSNorm and partial RoPE; the local output is gated by sigmoid(g_proj(h))
and projected by o_proj; global layers (6, 12, 18, 24, 30 of 32) attend over the whole prefix without a
gate. Hidden size 4096, 32 query heads and 8 KV heads of dim 128. Pre-LN (§3.1 "training
efficiency").

Readings: Pre-LN residual x <- x + o_proj(attn(RMSNorm(x))); input-norm weight
1, eps 1e-6; no biases; no MLP (the workload is attention-only); no final norm; weights are [out, in].

Parity pins (tests/test_stack_oracle.py): W_o = 0 leaves x unchanged; T = 1 closed form (one key, so
the attention output is v * sigmoid(g)); for T <= window a local layer with zero gate weights adds
exactly half of what the same layer run as a global layer adds; the layer schedule; the row-restricted
form (stack_layer_rows) equals the whole layer on every row.
"""
from __future__ import annotations

import numpy as np

from .attention import _attend_row, _sigmoid, key_set, prefill, qk_prologue
from .kv import is_global_layer


def layer_is_global(layer_1based: int, global_every: int = 6) -> bool:
    return is_global_layer(layer_1based, global_every)


def _rms_rows(x, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def stack_layer(x, w, *, is_global, n_q_heads=32, n_kv_heads=8, head_dim=128, window=128,
                rot_dim=42, rope_base=1e7, eps=1e-6, pos0=0):
    """One Pre-LN attention layer. x: [B, T, hidden] float64. w: dict of [out, in] float64 arrays
    'wq', 'wk', 'wv', 'wo' and, for local layers, 'wg'. Returns the updated residual stream."""
    B, T, Hd = x.shape
    h = _rms_rows(x, eps)
    q = (h @ w["wq"].T).reshape(B, T, n_q_heads, head_dim)
    k = (h @ w["wk"].T).reshape(B, T, n_kv_heads, head_dim)
    v = (h @ w["wv"].T).reshape(B, T, n_kv_heads, head_dim)
    if is_global:
        g = None
        a = prefill(q, k, v, None, window=0, gated=False, rot_dim=rot_dim, rope_base=rope_base,
                    eps=eps, pos0=pos0)
    else:
        g = (h @ w["wg"].T).reshape(B, T, n_q_heads, head_dim)
        a = prefill(q, k, v, g, window=window, gated=True, rot_dim=rot_dim, rope_base=rope_base,
                    eps=eps, pos0=pos0)
    return x + a.reshape(B, T, n_q_heads * head_dim) @ w["wo"].T


def stack_layer_rows(x, w, rows, *, is_global, n_q_heads=32, n_kv_heads=8, head_dim=128,
                     window=128, rot_dim=42, rope_base=1e7, eps=1e-6, pos0=0):
    """Rows `rows` of stack_layer's output for one sequence, x: [T, hidden] float64. The same steps
    as stack_layer, with the projections taken only where those rows need them: q (and the gate)
    of the rows themselves, k and v of the union of their key sets. Returns [len(rows), hidden]."""
    rows = [int(r) for r in rows]
    W = 0 if is_global else window
    keys = sorted(set().union(*(range(*key_set(t, W)) for t in rows)))
    at = {j: i for i, j in enumerate(keys)}
    hk = _rms_rows(x[keys], eps)
    kk = (hk @ w["wk"].T).reshape(len(keys), n_kv_heads, head_dim)
    vv = (hk @ w["wv"].T).reshape(len(keys), n_kv_heads, head_dim)
    khat = qk_prologue(kk, pos0 + np.asarray(keys), None, rot_dim=rot_dim, rope_base=rope_base,
                       eps=eps)
    hq = _rms_rows(x[rows], eps)
    q = (hq @ w["wq"].T).reshape(len(rows), n_q_heads, head_dim)
    g = None if is_global else (hq @ w["wg"].T).reshape(len(rows), n_q_heads, head_dim)
    scale = 1.0 / np.sqrt(head_dim)
    out = np.empty((len(rows), x.shape[1]), dtype=np.float64)
    for i, t in enumerate(rows):
        lo, hi = key_set(t, W)
        sel = [at[j] for j in range(lo, hi)]
        qhat = qk_prologue(q[i], pos0 + t, None, rot_dim=rot_dim, rope_base=rope_base, eps=eps)
        o = _attend_row(qhat, khat[sel], vv[sel], scale)
        if not is_global:
            o = o * _sigmoid(g[i])
        out[i] = x[t] + o.reshape(-1) @ w["wo"].T
    return out


def stack(x0, layer_weights, *, global_every=6, **kw):
    """Run the layers in order. layer_weights: iterable of per-layer weight dicts (1-indexed order).
    Layer l is global iff l % global_every == 0."""
    x = np.asarray(x0, dtype=np.float64)
    for l, w in enumerate(layer_weights, start=1):
        x = stack_layer(x, w, is_global=layer_is_global(l, global_every), **kw)
    return x
