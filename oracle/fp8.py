"""E4M3 value set, rounding, and decode over a KV cache stored in E4M3. TEST INFRASTRUCTURE ONLY.

The pages run their matrix multiplications in mixed FP8, with the E4M3 format on the forward pass
(ZGCM-1 zh-TW translation page, §3.1 "General pre-training", hyper-parameters; English page,
training-efficiency paragraph). Here the format stores the decode KV cache.

E4M3 is the OCP 8-bit floating-point format with a sign bit, 4 exponent bits (bias 7) and 3 mantissa
bits and no infinities: exponent field e = 1..15 with mantissa m = 0..7 encodes (1 + m/8) * 2^(e-7),
except e = 15, m = 7, which is NaN; e = 0 encodes the subnormals m/8 * 2^-6. The largest finite
value is 448, the smallest subnormal 2^-9.

Reading: values are rounded to the nearest E4M3 value, ties to the even
mantissa, and saturate at +-448.

Pins (tests/test_fp8_oracle.py): the value set has 127 non-negative members with the extremes
above; every member is a fixed point; midpoints round to the even neighbour; agreement with torch's
float8_e4m3fn cast (a library routine) on random values in range; the rounding error is at most half
a spacing; decode over the cache is invariant under a power-of-two change of scale, and writes the
rounded k_hat / v of the new token.
"""
from __future__ import annotations

import numpy as np

from .attention import _attend_row, _sigmoid, key_set, qk_prologue

E4M3_MAX = 448.0


def e4m3_values() -> np.ndarray:
    """All finite non-negative E4M3 values, ascending, from the field definition."""
    vals = [m / 8.0 * 2.0 ** -6 for m in range(8)]                      # e = 0: zero, subnormals
    for e in range(1, 16):
        for m in range(8):
            if e == 15 and m == 7:
                continue                                                  # NaN
            vals.append((1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(sorted(vals), dtype=np.float64)


def round_e4m3(x) -> np.ndarray:
    """Nearest E4M3 value of each element (ties to even mantissa), saturating at +-448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # spacing of the binade holding a: 2^(e - 3) for normals (e = floor(log2 a) >= -6), 2^-9 below
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    spacing = 2.0 ** (np.minimum(e, 8.0) - 3.0)
    r = np.round(a / spacing) * spacing          # np.round: half to even; a/spacing is exact
    return np.sign(x) * np.minimum(r, E4M3_MAX)


def decode_fp8_cache(q_new, k_new, v_new, gate, k_cache, v_cache, seqlens, *, k_scale, v_scale,
                     window, gated, rot_dim=42, rope_base=1e7, eps=1e-6, q_norm_w=None,
                     k_norm_w=None, scale=None):
    """One decode step over K/V caches whose entries are E4M3 values c standing for c * k_scale and
    c * v_scale. The new token's k_hat / k_scale and v / v_scale are rounded to E4M3 and written to
    their row (ring slot pos % window, or row pos); then the query attends as in decode().

    Caches are given and returned in E4M3 value units: [B, R, Hkv, D]. Returns (out [B, Hq, D],
    k_cache', v_cache')."""
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
        kc[b, slots[-1]] = round_e4m3(khat / k_scale)
        vc[b, slots[-1]] = round_e4m3(np.asarray(v_new[b], np.float64) / v_scale)
        o = _attend_row(qhat, kc[b, slots] * k_scale, vc[b, slots] * v_scale, scale)
        if gated:
            o = o * _sigmoid(np.asarray(gate[b], dtype=np.float64))
        out[b] = o
    return out, kc, vc
