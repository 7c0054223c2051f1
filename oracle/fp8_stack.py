"""E4M3 rows with per-row scales, the scaled E4M3 GEMM, and one attention layer whose projections run
on E4M3 operands. TEST INFRASTRUCTURE ONLY.

The pages train the model's forward matrix multiplications in FP8 with the E4M3 format (ZGCM-1
zh-TW translation page, §3.1 pre-training setup). Here that format carries the layer's projections:
the normalised hidden state, the weights and the attention output become E4M3 rows with one scale
each, and the products are exact sums of E4M3 values times the two scales.

Definitions (the readings, stated once here and in the library header):

* E4M3 is the OCP format of ``fp8.py`` (codes 0x00-0x7E non-negative, ascending; bit 7 the sign;
  0x7F and 0xFF NaN).
* A row h is quantized with amax = max |h|: scale = amax / 448 and values E4M3(h * (448 / amax)),
  every step in fp32 arithmetic as written (each of the two divisions and the product rounded to
  fp32 once), the E4M3 rounding to nearest with ties to the even mantissa; a row of zeros gets
  scale 1 and zero values. The row then stands for its values times its scale.
* The layer: h = RMSNorm(x) (fp64, weight 1), its rows quantized from fp32(h); q, k, v and the gate
  are the dequantized h times the dequantized weights (weights quantized per output row); the
  attention is ``prefill`` in fp64; its output rows are quantized and the output projection adds
  their dequantized product with the dequantized W_o to x. Nothing else is rounded.

Pins (tests/test_fp8_stack_oracle.py): decoding every code against the value set built from the
field definition; quantization of a zero row, the row maximum landing on +-448, the half-spacing
error bound, exact round trips of rows that are already E4M3 values, and agreement with torch's
float8_e4m3fn cast (a library routine) of the same fp32 products; the GEMM against a brute-force
triple loop; the row-restricted layer equal to the whole layer on every row; a zero output
projection leaving x unchanged.
"""
from __future__ import annotations

import numpy as np

from .attention import _attend_row, _sigmoid, key_set, prefill, qk_prologue
from .fp8 import E4M3_MAX, round_e4m3
from .kv import is_global_layer

_F32_MAX = np.float32(E4M3_MAX)


def e4m3_decode(codes) -> np.ndarray:
    """Values of E4M3 codes (uint8) from the field definition: sign bit 7, exponent bits 6-3 (bias
    7), mantissa bits 2-0; exponent 0 holds the subnormals m/8 * 2^-6; 0x7F / 0xFF are NaN."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def quant_rows_e4m3(x):
    """Rows of x (last axis) as E4M3 values and fp32 scales, in the fp32 arithmetic the definition
    states. x is taken as fp32 (callers pass fp32 values or values that fp32 holds exactly).
    Returns (values fp64 [..., dim], scale fp32 [...])."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    pos = amax > 0
    safe = np.where(pos, amax, np.float32(1.0)).astype(np.float32)
    inv = np.where(pos, _F32_MAX / safe, np.float32(0.0)).astype(np.float32)
    scale = np.where(pos, safe / _F32_MAX, np.float32(1.0)).astype(np.float32)
    prod = (x32 * inv[..., None]).astype(np.float32)
    return round_e4m3(prod.astype(np.float64)), scale


def gemm_e4m3(xv, xs, wv, ws):
    """Y = diag(xs) Xv Wv^T diag(ws) in fp64 for E4M3 values Xv [M, K], Wv [N, K]."""
    xv = np.asarray(xv, np.float64)
    wv = np.asarray(wv, np.float64)
    return (xv @ wv.T) * np.asarray(xs, np.float64)[:, None] * np.asarray(ws, np.float64)[None, :]


def quantize_layer_weights(w):
    """Per-output-row E4M3 values and scales of a layer's weight dict (bf16 values as fp64):
    {name: (values, scale)} for 'wq', 'wk', 'wv', 'wo' and 'wg' when present."""
    return {n: quant_rows_e4m3(np.asarray(a, np.float64)) for n, a in w.items()}


def _deq(vs):
    v, s = vs
    return v * np.asarray(s, np.float64)[..., None]


def _rms_rows(x, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def stack_layer_fp8(x, wf, *, is_global, n_q_heads=32, n_kv_heads=8, head_dim=128, window=128,
                    rot_dim=42, rope_base=1e7, eps=1e-6, pos0=0):
    """One Pre-LN attention layer with E4M3 projections. x: [B, T, hidden] float64; wf: the output of
    quantize_layer_weights. Returns the updated residual stream."""
    B, T, Hd = x.shape
    hd = _deq(quant_rows_e4m3(_rms_rows(x, eps)))
    q = (hd @ _deq(wf["wq"]).T).reshape(B, T, n_q_heads, head_dim)
    k = (hd @ _deq(wf["wk"]).T).reshape(B, T, n_kv_heads, head_dim)
    v = (hd @ _deq(wf["wv"]).T).reshape(B, T, n_kv_heads, head_dim)
    if is_global:
        a = prefill(q, k, v, None, window=0, gated=False, rot_dim=rot_dim, rope_base=rope_base,
                    eps=eps, pos0=pos0)
    else:
        g = (hd @ _deq(wf["wg"]).T).reshape(B, T, n_q_heads, head_dim)
        a = prefill(q, k, v, g, window=window, gated=True, rot_dim=rot_dim, rope_base=rope_base,
                    eps=eps, pos0=pos0)
    ad = _deq(quant_rows_e4m3(a.reshape(B, T, n_q_heads * head_dim)))
    return x + ad @ _deq(wf["wo"]).T


def stack_layer_rows_fp8(x, wf, rows, *, is_global, n_q_heads=32, n_kv_heads=8, head_dim=128,
                         window=128, rot_dim=42, rope_base=1e7, eps=1e-6, pos0=0):
    """Rows `rows` of stack_layer_fp8's output for one sequence, x: [T, hidden] float64. Every
    quantization is per row, so only the rows a sampled output needs are projected: q (and the
    gate) of the rows themselves, k and v of the union of their key sets."""
    rows = [int(r) for r in rows]
    W = 0 if is_global else window
    keys = sorted(set().union(*(range(*key_set(t, W)) for t in rows)))
    at = {j: i for i, j in enumerate(keys)}
    hk = _deq(quant_rows_e4m3(_rms_rows(x[keys], eps)))
    kk = (hk @ _deq(wf["wk"]).T).reshape(len(keys), n_kv_heads, head_dim)
    vv = (hk @ _deq(wf["wv"]).T).reshape(len(keys), n_kv_heads, head_dim)
    khat = qk_prologue(kk, pos0 + np.asarray(keys), None, rot_dim=rot_dim, rope_base=rope_base,
                       eps=eps)
    hq = _deq(quant_rows_e4m3(_rms_rows(x[rows], eps)))
    q = (hq @ _deq(wf["wq"]).T).reshape(len(rows), n_q_heads, head_dim)
    g = None if is_global else (hq @ _deq(wf["wg"]).T).reshape(len(rows), n_q_heads, head_dim)
    scale = 1.0 / np.sqrt(head_dim)
    a = np.empty((len(rows), n_q_heads * head_dim), dtype=np.float64)
    for i, t in enumerate(rows):
        lo, hi = key_set(t, W)
        sel = [at[j] for j in range(lo, hi)]
        qhat = qk_prologue(q[i], pos0 + t, None, rot_dim=rot_dim, rope_base=rope_base, eps=eps)
        o = _attend_row(qhat, khat[sel], vv[sel], scale)
        if not is_global:
            o = o * _sigmoid(g[i])
        a[i] = o.reshape(-1)
    return x[rows] + _deq(quant_rows_e4m3(a)) @ _deq(wf["wo"]).T


def stack_fp8(x0, layer_weights_fp8, *, global_every=6, **kw):
    """The layers in order, each with E4M3 projections (layer l global iff l % global_every == 0)."""
    x = np.asarray(x0, dtype=np.float64)
    for l, wf in enumerate(layer_weights_fp8, start=1):
        x = stack_layer_fp8(x, wf, is_global=is_global_layer(l, global_every), **kw)
    return x
