"""Pin the attention oracle to an independent pure-Python scalar formulation on tiny shapes.

The brute force below writes every step out with scalar loops: RMSNorm with math.sqrt, RoPE as a
complex multiplication by exp(i*phi), the causal/window mask as a predicate on (i, j), the GQA head map
as h*Hkv//Hq, softmax with math.exp. A dropped term, wrong sign, transposed index or off-by-one in the
oracle's vectorised code fails here to 1e-12.
"""
import cmath
import math

import numpy as np
import pytest

import oracle


def _brute(q, k, v, gate, W, gated, rot_dim, base, eps, qw, kw, pos0):
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    half = rot_dim // 2

    def norm_rope(x, w, pos):
        x = [float(a) for a in x]
        ms = sum(a * a for a in x) / len(x)
        r = 1.0 / math.sqrt(ms + eps)
        y = [x[d] * r * (1.0 if w is None else float(w[d])) for d in range(len(x))]
        for i in range(half):
            z = complex(y[i], y[i + half]) * cmath.exp(1j * pos * base ** (-2.0 * i / rot_dim))
            y[i], y[i + half] = z.real, z.imag
        return y

    out = np.zeros(q.shape)
    for b in range(B):
        khat = [[norm_rope(k[b, j, g], kw, pos0 + j) for g in range(Hkv)] for j in range(T)]
        for i in range(T):
            for h in range(Hq):
                g = h * Hkv // Hq
                qh = norm_rope(q[b, i, h], qw, pos0 + i)
                allowed = [j for j in range(T) if j <= i and (W <= 0 or i - j < W)]
                s = [sum(qh[d] * khat[j][g][d] for d in range(D)) / math.sqrt(D) for j in allowed]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                z = sum(e)
                for d in range(D):
                    o = sum(e[n] / z * float(v[b, j, g, d]) for n, j in enumerate(allowed))
                    if gated:
                        o *= 1.0 / (1.0 + math.exp(-float(gate[b, i, h, d])))
                    out[b, i, h, d] = o
    return out


CASES = [
    # B, T, Hq, Hkv, D, W, gated, rot_dim, base, pos0
    (1, 1, 4, 1, 8, 4, True, 4, 1e4, 0),
    (1, 2, 4, 1, 8, 1, True, 4, 1e4, 0),
    (2, 5, 4, 1, 16, 2, True, 6, 1e4, 0),
    (1, 7, 8, 2, 16, 3, False, 6, 100.0, 3),
    (2, 6, 8, 2, 12, 0, False, 4, 1e6, 0),
    (1, 9, 4, 2, 10, 4, True, 10, 1e4, 5),
    (1, 6, 4, 1, 8, 128, True, 2, 1e4, 0),
    (1, 5, 32, 8, 8, 2, True, 2, 1e7, 17),
]


@pytest.mark.parametrize("B,T,Hq,Hkv,D,W,gated,rot_dim,base,pos0", CASES)
def test_prefill_matches_bruteforce(B, T, Hq, Hkv, D, W, gated, rot_dim, base, pos0):
    rng = np.random.default_rng(B * 1000 + T * 10 + D)
    q = rng.standard_normal((B, T, Hq, D))
    k = rng.standard_normal((B, T, Hkv, D))
    v = rng.standard_normal((B, T, Hkv, D))
    g = rng.standard_normal((B, T, Hq, D))
    qw = rng.uniform(0.5, 2.0, D)
    kw = rng.uniform(0.5, 2.0, D)
    eps = 1e-6
    ref = _brute(q, k, v, g, W, gated, rot_dim, base, eps, qw, kw, pos0)
    got = oracle.prefill(q, k, v, g, window=W, gated=gated, rot_dim=rot_dim, rope_base=base,
                         eps=eps, q_norm_w=qw, k_norm_w=kw, pos0=pos0)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_decode_matches_bruteforce_row():
    """Decode at position pos equals the brute-force prefill row pos (ring and linear caches)."""
    rng = np.random.default_rng(7)
    B, T, Hq, Hkv, D, rot, base, eps = 2, 9, 8, 2, 12, 6, 1e4, 1e-6
    q = rng.standard_normal((B, T, Hq, D))
    k = rng.standard_normal((B, T, Hkv, D))
    v = rng.standard_normal((B, T, Hkv, D))
    g = rng.standard_normal((B, T, Hq, D))
    for W in (4, 0):
        ref = _brute(q, k, v, g, W, W > 0, rot, base, eps, None, None, 0)
        seqlens = np.array([T, T - 3])
        rows = W if W > 0 else T
        kc = np.zeros((B, rows, Hkv, D))
        vc = np.zeros((B, rows, Hkv, D))
        for b in range(B):
            pos = seqlens[b] - 1
            for p in range(max(0, pos - W + 1) if W > 0 else 0, pos):
                slot = p % W if W > 0 else p
                kh = oracle.qk_prologue(k[b, p], p, None, rot_dim=rot, rope_base=base, eps=eps)
                kc[b, slot] = kh
                vc[b, slot] = v[b, p]
        qn = np.stack([q[b, seqlens[b] - 1] for b in range(B)])
        kn = np.stack([k[b, seqlens[b] - 1] for b in range(B)])
        vn = np.stack([v[b, seqlens[b] - 1] for b in range(B)])
        gn = np.stack([g[b, seqlens[b] - 1] for b in range(B)])
        out, _, _ = oracle.decode(qn, kn, vn, gn, kc, vc, seqlens, window=W, gated=W > 0,
                                  rot_dim=rot, rope_base=base, eps=eps)
        for b in range(B):
            np.testing.assert_allclose(out[b], ref[b, seqlens[b] - 1], rtol=0, atol=1e-12)
