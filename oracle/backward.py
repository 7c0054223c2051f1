"""fp64 backward of one attention layer (prefill): gradients of q, k, v and the gate logits.
TEST INFRASTRUCTURE ONLY.

The pages' throughput figures are training figures (ZGCM-1 zh-TW translation page, §2.2: tokens per
second per GPU while pre-training the attention schedules; §3.1: pre-training), so the layer's
backward pass sits next to its forward. The forward is the plain definition of oracle.attention
(QK-RMSNorm with weight 1, partial RoPE, banded or full causal GQA softmax attention, sigmoid gate);
this module applies the chain rule to it, step by step in the reverse order, for the scalar
L = sum(dy * y) with y the layer output.

Steps, per sequence (h a query head, t a query, j a key, G query heads per key/value head):
  gate      y = o * s, s = sigmoid(g):  do = dy * s,  dg = dy * o * s * (1 - s)
  values    dv[j] = sum over the group's (h, t) of p[h, t, j] * do[h, t]
  softmax   dp[h, t, j] = do[h, t] . v[j];  ds = p * (dp - sum_j p * dp)   (masked keys: p = 0)
  scores    s = scale * q_hat . k_hat:  dq_hat = scale * ds k_hat,  dk_hat = scale * ds^T q_hat
  RoPE      x_hat = R(pos) x_n (a rotation of each pair):  dx_n = R(pos)^T dx_hat
  RMSNorm   x_n = x / r, r = sqrt(mean(x^2) + eps):  dx = (dx_n - x_n * mean(dx_n * x_n)) / r

Pin (tests/test_backward_oracle.py): central finite differences of sum(dy * forward) with the
forward oracle, on small shapes, for every input.
"""
from __future__ import annotations

import numpy as np

from .attention import _sigmoid, key_set, partial_rope, qk_prologue


def _rms_norm_backward(x, dxn, eps):
    """Gradient through x_n = x / sqrt(mean(x^2) + eps) over the last axis."""
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    xn = x / r
    return (dxn - xn * np.mean(dxn * xn, axis=-1, keepdims=True)) / r


def _prologue_backward(x, pos, dxhat, *, rot_dim, rope_base, eps):
    """Gradient through x_hat = RoPE(RMSNorm(x)) at positions pos: RoPE's transpose is the
    rotation by the negated angle."""
    dxn = partial_rope(dxhat, -np.asarray(pos, dtype=np.float64), rot_dim, rope_base)
    return _rms_norm_backward(np.asarray(x, dtype=np.float64), dxn, eps)


def layer_backward(q, k, v, gate, dy, *, window, gated, rot_dim=42, rope_base=1e4, eps=1e-6,
                   scale=None, pos0=0):
    """q, gate, dy: [B, T, Hq, D]; k, v: [B, T, Hkv, D]. Returns (dq, dk, dv, dgate) of
    L = sum(dy * y); dgate is None when not gated."""
    q, k, v, dy = (np.asarray(a, dtype=np.float64) for a in (q, k, v, dy))
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    pos = pos0 + np.arange(T)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dg = np.zeros_like(q) if gated else None
    mask = np.zeros((T, T), dtype=bool)
    for t in range(T):
        lo, hi = key_set(t, window)
        mask[t, lo:hi] = True
    for b in range(B):
        qh = qk_prologue(q[b], pos, None, rot_dim=rot_dim, rope_base=rope_base, eps=eps)  # [T,Hq,D]
        kh = qk_prologue(k[b], pos, None, rot_dim=rot_dim, rope_base=rope_base, eps=eps)  # [T,Hkv,D]
        dqh, dkh = np.zeros_like(qh), np.zeros_like(kh)
        for h in range(Hq):
            c = h // G
            s = scale * qh[:, h, :] @ kh[:, c, :].T                       # [T, T]
            s = np.where(mask, s, -np.inf)
            p = np.exp(s - np.max(s, axis=1, keepdims=True))
            p = p / np.sum(p, axis=1, keepdims=True)                       # [T, T]
            o = p @ v[b, :, c, :]                                          # [T, D]
            if gated:
                sg = _sigmoid(np.asarray(gate[b, :, h, :], dtype=np.float64))
                do = dy[b, :, h, :] * sg
                dg[b, :, h, :] = dy[b, :, h, :] * o * sg * (1.0 - sg)
            else:
                do = dy[b, :, h, :]
            dv[b, :, c, :] += p.T @ do
            dp = do @ v[b, :, c, :].T                                      # [T, T]
            ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
            dqh[:, h, :] = scale * ds @ kh[:, c, :]
            dkh[:, c, :] += scale * ds.T @ qh[:, h, :]
        dq[b] = _prologue_backward(q[b], pos, dqh, rot_dim=rot_dim, rope_base=rope_base, eps=eps)
        dk[b] = _prologue_backward(k[b], pos, dkh, rot_dim=rot_dim, rope_base=rope_base, eps=eps)
    return dq, dk, dv, dg


def row_lse(q, k, *, window, rot_dim=42, rope_base=1e4, eps=1e-6, scale=None, pos0=0):
    """Natural-log log-sum-exp of each query row's scaled scores: [B, T, Hq]."""
    q, k = np.asarray(q, np.float64), np.asarray(k, np.float64)
    B, T, Hq, D = q.shape
    G = Hq // k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    pos = pos0 + np.arange(T)
    out = np.zeros((B, T, Hq))
    for b in range(B):
        qh = qk_prologue(q[b], pos, None, rot_dim=rot_dim, rope_base=rope_base, eps=eps)
        kh = qk_prologue(k[b], pos, None, rot_dim=rot_dim, rope_base=rope_base, eps=eps)
        for t in range(T):
            lo, hi = key_set(t, window)
            s = scale * np.stack([kh[lo:hi, h // G] @ qh[t, h] for h in range(Hq)])  # [Hq, n]
            m = np.max(s, axis=1)
            out[b, t] = m + np.log(np.sum(np.exp(s - m[:, None]), axis=1))
    return out


def layer_backward_rows(q, k, v, gate, dy, *, window, gated, q_rows, k_rows, rot_dim=42,
                        rope_base=1e4, eps=1e-6, scale=None, pos0=0):
    """The gradients of layer_backward for ONE sequence, evaluated only where asked: dq (and
    dgate) at query rows `q_rows`, dk and dv at key rows `k_rows`, plus the natural-log row
    log-sum-exp at `q_rows`. q, gate, dy: [T, Hq, D]; k, v: [T, Hkv, D] (any float dtype, widened
    to fp64 row by row). Same chain rule as layer_backward, restricted to the rows it touches:

      dq[t]  needs row t's softmax (its key set), dP[t, j] = dO[t] . v[j] and D[t] = sum_j P dP;
      dk[j], dv[j] sum over the queries t whose key set holds j (t in [j, j + W) or [j, T)), each
             needing its own full softmax row and D[t].

    Returns (dq [len(q_rows), Hq, D], dk [len(k_rows), Hkv, D], dv [len(k_rows), Hkv, D],
    dgate [len(q_rows), Hq, D] or None, lse [len(q_rows), Hq])."""
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    f64 = lambda a: np.asarray(a, dtype=np.float64)
    q_rows = [int(t) for t in q_rows]
    k_rows = [int(j) for j in k_rows]

    # queries whose softmax rows are needed, and the keys those rows read
    need_t = set(q_rows)
    for j in k_rows:
        hi = min(T, j + window) if window > 0 else T
        need_t.update(range(j, hi))
    need_t = sorted(need_t)
    k_lo = min(key_set(t, window)[0] for t in need_t)
    k_hi = max(need_t) + 1
    keys = np.arange(k_lo, k_hi)
    kh = qk_prologue(f64(k[k_lo:k_hi]), pos0 + keys, None, rot_dim=rot_dim, rope_base=rope_base,
                     eps=eps)                                              # [nk, Hkv, D]
    vk = f64(v[k_lo:k_hi])

    rows = {}  # t -> (qhat [Hq, D], P [Hq, n], dO [Hq, D], dS [Hq, n], lo, o [Hq, D])
    for t in need_t:
        lo, hi = key_set(t, window)
        qh = qk_prologue(f64(q[t])[None], np.array([pos0 + t]), None, rot_dim=rot_dim,
                         rope_base=rope_base, eps=eps)[0]                  # [Hq, D]
        P = np.empty((Hq, hi - lo))
        o = np.empty((Hq, D))
        dO = f64(dy[t]).copy()
        dP = np.empty((Hq, hi - lo))
        for h in range(Hq):
            c = h // G
            s = scale * kh[lo - k_lo:hi - k_lo, c] @ qh[h]
            m = s.max()
            e = np.exp(s - m)
            P[h] = e / e.sum()
            o[h] = P[h] @ vk[lo - k_lo:hi - k_lo, c]
        if gated:
            sg = _sigmoid(f64(gate[t]))
            dO = dO * sg
        for h in range(Hq):
            dP[h] = vk[lo - k_lo:hi - k_lo, h // G] @ dO[h]
        Dt = np.sum(P * dP, axis=1, keepdims=True)
        rows[t] = (qh, P, dO, P * (dP - Dt), lo, o)

    dq = np.empty((len(q_rows), Hq, D))
    dg = np.empty((len(q_rows), Hq, D)) if gated else None
    lse = np.empty((len(q_rows), Hq))
    for n, t in enumerate(q_rows):
        qh, P, dO, dS, lo, o = rows[t]
        hi = t + 1
        dqh = np.stack([scale * dS[h] @ kh[lo - k_lo:hi - k_lo, h // G] for h in range(Hq)])
        dq[n] = _prologue_backward(f64(q[t])[None], np.array([pos0 + t]), dqh[None],
                                   rot_dim=rot_dim, rope_base=rope_base, eps=eps)[0]
        for h in range(Hq):
            s = scale * kh[lo - k_lo:hi - k_lo, h // G] @ qh[h]
            lse[n, h] = s.max() + np.log(np.sum(np.exp(s - s.max())))
        if gated:
            sg = _sigmoid(f64(gate[t]))
            dg[n] = f64(dy[t]) * o * sg * (1.0 - sg)

    dk = np.zeros((len(k_rows), Hkv, D))
    dv = np.zeros((len(k_rows), Hkv, D))
    for n, j in enumerate(k_rows):
        dkh = np.zeros((Hkv, D))
        hi = min(T, j + window) if window > 0 else T
        for t in range(j, hi):
            qh, P, dO, dS, lo, _ = rows[t]
            for h in range(Hq):
                c = h // G
                dv[n, c] += P[h, j - lo] * dO[h]
                dkh[c] += scale * dS[h, j - lo] * qh[h]
        dk[n] = _prologue_backward(f64(k[j])[None], np.array([pos0 + j]), dkh[None],
                                   rot_dim=rot_dim, rope_base=rope_base, eps=eps)[0]
    return dq, dk, dv, dg, lse
