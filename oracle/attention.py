"""fp64 oracle: QK-RMSNorm, partial RoPE, banded / full causal GQA attention, sigmoid gate, decode.

TEST INFRASTRUCTURE ONLY (see the package docstring). Plain NumPy float64 throughout.

What the pages fix (ZGCM-1 zh-TW translation page, §2.1 "Model overview" and Fig. 3; zh-CN tutorial
page, architecture paragraph):
  * 32 query heads, 8 key/value heads (GQA), head dim 128;
  * local layers attend over a 128-token sliding window, global layers over the whole causal prefix;
  * q and k are normalised with RMSNorm and rotated with partial RoPE (rotary fraction 0.33);
  * the local output is multiplied elementwise by sigmoid(g_proj(h)) before o_proj; global layers
    have no gate.

Readings taken where the pages are silent:
  * RMSNorm is per head over the 128 head dims with one shared weight vector for q and one for k;
  * RMSNorm is applied before RoPE (the order in which Fig. 3 lists them);
  * rot_dim = floor(0.33 * 128) = 42; rotate-half pairing (i, i + rot_dim/2), frequency
    theta_i = base^(-2i/rot_dim); dims >= rot_dim pass through;
  * positions are 0-based (pos0 + t); softmax scale 1/sqrt(head_dim);
  * window W keeps key j for query i iff i - W < j <= i (W keys including the query itself);
  * query head h reads key/value head floor(h / (Hq/Hkv)).

Parity pins (tests/test_oracle_*.py): pure-Python brute force on tiny shapes with a complex-number
RoPE; torch fp64 SDPA with an explicit band mask; W >= T equals full causal; zero gate logit gives
exactly half the ungated output; probabilities sum to 1; V == 1 gives O == 1; pair norms preserved by
RoPE; relative-position (shift) invariance of scores; RMSNorm mean-square identity; single-key and
uniform-key closed forms; decode equals the matching prefill row; ring-slot permutation invariance.
"""
from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------------------------- norm
def rms_norm(x: np.ndarray, w: np.ndarray | None, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x * w / sqrt(mean(x^2) + eps).

    QK normalisation "implemented with RMSNorm" (ZGCM-1 zh-TW translation, §2.1); the per-head axis
    is the reading stated in the module header."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    y = x / np.sqrt(ms + eps)
    if w is not None:
        y = y * np.asarray(w, dtype=np.float64)
    return y


# --------------------------------------------------------------------------------------------- rope
def rope_inv_freq(rot_dim: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/rot_dim) for i < rot_dim/2 (partial RoPE, ZGCM-1 zh-TW §2.1; base 1e7 at
    256K per §3.2)."""
    half = rot_dim // 2
    i = np.arange(half, dtype=np.float64)
    return np.power(float(base), -2.0 * i / float(rot_dim))


def partial_rope(x: np.ndarray, pos: np.ndarray, rot_dim: int, base: float) -> np.ndarray:
    """Rotate dims [0, rot_dim) of the last axis by position-dependent angles; keep the rest.

    x: [..., N, H, D] with pos: [N] (positions of axis -3), or x: [H, D] with a scalar pos.
    Pair (i, i + rot_dim/2) is rotated by phi = pos * theta_i:
        (a, c) -> (a cos phi - c sin phi, c cos phi + a sin phi).
    """
    x = np.asarray(x, dtype=np.float64)
    if rot_dim == 0:
        return x.copy()
    half = rot_dim // 2
    theta = rope_inv_freq(rot_dim, base)                       # [half]
    pos = np.asarray(pos, dtype=np.float64)
    if pos.ndim == 0:
        phi = pos * theta                                      # [half]
        cos, sin = np.cos(phi), np.sin(phi)                    # broadcast over [H, half]
    else:
        phi = pos[:, None] * theta[None, :]                    # [N, half]
        cos = np.cos(phi)[:, None, :]                          # [N, 1, half] over heads
        sin = np.sin(phi)[:, None, :]
    out = x.copy()
    a = x[..., :half]
    c = x[..., half:rot_dim]
    out[..., :half] = a * cos - c * sin
    out[..., half:rot_dim] = c * cos + a * sin
    return out


def qk_prologue(x, pos, w, *, rot_dim, rope_base, eps):
    """RMSNorm then partial RoPE (the order of Fig. 3's q/k branches)."""
    return partial_rope(rms_norm(x, w, eps), pos, rot_dim, rope_base)


# ------------------------------------------------------------------------------------------ masking
def key_set(t: int, window: int) -> tuple[int, int]:
    """Half-open key range [lo, t+1) of query t: the last `window` tokens up to and including t
    (sliding window, ZGCM-1 zh-TW §2.1), or the whole prefix when window <= 0 (global causal)."""
    lo = max(0, t - window + 1) if window > 0 else 0
    return lo, t + 1


def _sigmoid(g):
    return 1.0 / (1.0 + np.exp(-g))


def _softmax_last(s):
    s = s - np.max(s, axis=-1, keepdims=True)
    p = np.exp(s)
    return p / np.sum(p, axis=-1, keepdims=True)


# ------------------------------------------------------------------------------------------ prefill
def attention_probs_row(qhat_t, khat_keys, scale):
    """Softmax probabilities of one query row.

    qhat_t: [Hq, D]; khat_keys: [n, Hkv, D]. Returns p: [Hq, n] (GQA: head h uses kv head h // G)."""
    hq, d = qhat_t.shape
    hkv = khat_keys.shape[1]
    g = hq // hkv
    qg = qhat_t.reshape(hkv, g, d)                                 # [Hkv, G, D]
    kk = np.transpose(khat_keys, (1, 2, 0))                        # [Hkv, D, n]
    s = np.matmul(qg, kk) * scale                                  # [Hkv, G, n]
    return _softmax_last(s).reshape(hq, -1)


def _attend_row(qhat_t, khat_keys, v_keys, scale):
    hq, d = qhat_t.shape
    hkv = khat_keys.shape[1]
    g = hq // hkv
    p = attention_probs_row(qhat_t, khat_keys, scale).reshape(hkv, g, -1)   # [Hkv, G, n]
    vv = np.transpose(v_keys, (1, 0, 2))                                     # [Hkv, n, D]
    return np.matmul(p, vv).reshape(hq, d)


def prefill_rows(q, k, v, gate, rows, *, window, gated, rot_dim=42, rope_base=1e4, eps=1e-6,
                 q_norm_w=None, k_norm_w=None, scale=None, pos0=0, batches=None):
    """Attention output of selected query rows.

    q, gate: [B, T, Hq, D]; k, v: [B, T, Hkv, D] (fp64 widening of the inputs). rows: iterable of
    query indices. Returns [len(batches), len(rows), Hq, D] float64.

    Steps per (b, t): q_hat = RoPE(RMSNorm(q)), k_hat = RoPE(RMSNorm(k)) at positions pos0 + t;
    s_j = q_hat . k_hat_j * scale over the key set; p = softmax(s); o = sum_j p_j v_j; if gated,
    o *= sigmoid(gate) elementwise (ZGCM-1 zh-TW §2.1 Fig. 3: GatedSWA(h) = o_proj(A(q,k,v) *
    sigmoid(g_proj(h))))."""
    B, T, Hq, D = q.shape
    rows = [int(r) for r in rows]
    batches = list(range(B)) if batches is None else [int(b) for b in batches]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((len(batches), len(rows), Hq, D), dtype=np.float64)
    if not rows:
        return out
    lo_all = min(key_set(t, window)[0] for t in rows)
    hi_all = max(rows) + 1
    for bi, b in enumerate(batches):
        kpos = pos0 + np.arange(lo_all, hi_all)
        khat = qk_prologue(np.asarray(k[b, lo_all:hi_all], dtype=np.float64), kpos, k_norm_w,
                           rot_dim=rot_dim, rope_base=rope_base, eps=eps)       # [n, Hkv, D]
        vb = np.asarray(v[b, lo_all:hi_all], dtype=np.float64)
        for ri, t in enumerate(rows):
            lo, hi = key_set(t, window)
            qhat = qk_prologue(np.asarray(q[b, t], dtype=np.float64), pos0 + t, q_norm_w,
                               rot_dim=rot_dim, rope_base=rope_base, eps=eps)    # [Hq, D]
            o = _attend_row(qhat, khat[lo - lo_all:hi - lo_all], vb[lo - lo_all:hi - lo_all], scale)
            if gated:
                o = o * _sigmoid(np.asarray(gate[b, t], dtype=np.float64))
            out[bi, ri] = o
    return out


def prefill(q, k, v, gate, **kw):
    """All rows of every sequence: [B, T, Hq, D] float64 (see prefill_rows)."""
    T = q.shape[1]
    return prefill_rows(q, k, v, gate, range(T), **kw)


# ------------------------------------------------------------------------------------------- decode
def decode(q_new, k_new, v_new, gate, k_cache, v_cache, seqlens, *, window, gated, rot_dim=42,
           rope_base=1e7, eps=1e-6, q_norm_w=None, k_norm_w=None, scale=None):
    """One decode step per sequence over a KV cache of post-norm/RoPE keys.

    q_new, gate: [B, Hq, D]; k_new, v_new: [B, Hkv, D]; caches [B, R, Hkv, D]; seqlens[b] = number of
    positions after appending, so the new token sits at pos = seqlens[b] - 1.
    window > 0: the cache is a ring of `window` slots and position p lives in slot p % window (the
    local layers keep a fixed 128-token window, ZGCM-1 zh-TW §2.3). window == 0: linear cache, row p.
    Returns (out [B, Hq, D], k_cache', v_cache') with the new k_hat / v written into their rows.
    The key set is the same as prefill row pos: positions max(0, pos - window + 1) .. pos."""
    B, Hq, D = q_new.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        pos = int(seqlens[b]) - 1
        qhat = qk_prologue(np.asarray(q_new[b], np.float64), pos, q_norm_w, rot_dim=rot_dim,
                           rope_base=rope_base, eps=eps)
        khat = qk_prologue(np.asarray(k_new[b], np.float64), pos, k_norm_w, rot_dim=rot_dim,
                           rope_base=rope_base, eps=eps)
        lo, hi = key_set(pos, window)
        positions = np.arange(lo, hi)
        slots = positions % window if window > 0 else positions
        new_row = slots[-1]
        kc[b, new_row] = khat
        vc[b, new_row] = np.asarray(v_new[b], np.float64)
        o = _attend_row(qhat, kc[b, slots], vc[b, slots], scale)
        if gated:
            o = o * _sigmoid(np.asarray(gate[b], dtype=np.float64))
        out[b] = o
    return out, kc, vc
