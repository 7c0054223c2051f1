"""Pins of the oracle's layer backward (oracle/backward.py): central finite differences of
sum(dy * y), y = the forward oracle's layer output, for every input, on small shapes (the chain rule
and the forward are written independently, so a dropped term, a wrong sign or a transposed operand
in the backward shows up as a mismatch). The log-sum-exp rows are pinned
two ways: against torch.logsumexp of scores built by an independent scalar formulation, and as the
normaliser that turns the scores back into the softmax rows behind the brute-force-pinned forward."""
import cmath
import math

import numpy as np
import pytest
import torch

import oracle


def _case(seed, B, T, Hq, Hkv, D, gated):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, Hq, D))
    k = rng.standard_normal((B, T, Hkv, D))
    v = rng.standard_normal((B, T, Hkv, D))
    g = rng.standard_normal((B, T, Hq, D)) if gated else None
    dy = rng.standard_normal((B, T, Hq, D))
    return q, k, v, g, dy


@pytest.mark.parametrize("window,gated,rot", [(0, False, 6), (3, True, 6), (4, True, 0), (2, False, 8)])
def test_backward_matches_finite_differences(window, gated, rot):
    B, T, Hq, Hkv, D = 2, 7, 4, 2, 16
    q, k, v, g, dy = _case(10 + window + rot, B, T, Hq, Hkv, D, gated)
    kw = dict(window=window, gated=gated, rot_dim=rot, rope_base=100.0, eps=1e-6, pos0=3)

    def loss(q_, k_, v_, g_):
        return float(np.sum(dy * oracle.prefill(q_, k_, v_, g_, **kw)))

    dq, dk, dv, dg = oracle.layer_backward(q, k, v, g, dy, **kw)
    rng = np.random.default_rng(99)
    h = 1e-6
    inputs = [("q", q, dq), ("k", k, dk), ("v", v, dv)] + ([("g", g, dg)] if gated else [])
    for name, x, grad in inputs:
        for _ in range(12):
            idx = tuple(rng.integers(0, n) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v, "g": g}
            args[name] = xp
            lp = loss(args["q"], args["k"], args["v"], args["g"])
            args[name] = xm
            lm = loss(args["q"], args["k"], args["v"], args["g"])
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def _scalar_scores(q, k, t, h, G, window, rot_dim, base, eps, scale):
    """Scores of query (t, h) written out with scalar loops and an independent prologue: RMSNorm
    with math.sqrt, RoPE as a complex multiplication by exp(i * pos * theta)."""
    half = rot_dim // 2

    def norm_rope(x, pos):
        x = [float(a) for a in x]
        r = 1.0 / math.sqrt(sum(a * a for a in x) / len(x) + eps)
        y = [a * r for a in x]
        for i in range(half):
            z = complex(y[i], y[i + half]) * cmath.exp(1j * pos * base ** (-2.0 * i / rot_dim))
            y[i], y[i + half] = z.real, z.imag
        return y

    qh = norm_rope(q[t, h], t)
    lo = max(0, t - window + 1) if window > 0 else 0
    return [scale * sum(a * b for a, b in zip(qh, norm_rope(k[j, h // G], j)))
            for j in range(lo, t + 1)]


@pytest.mark.parametrize("window", [3, 0])
def test_row_lse_matches_library_logsumexp(window):
    """row_lse against torch.logsumexp of scores built by the scalar formulation above."""
    q, k, _, _, _ = _case(5, 1, 9, 4, 2, 16, False)
    lse = oracle.row_lse(q, k, window=window, rot_dim=6, rope_base=100.0)
    for t in range(9):
        for h in range(4):
            s = torch.tensor(_scalar_scores(q[0], k[0], t, h, 2, window, 6, 100.0, 1e-6, 0.25),
                             dtype=torch.float64)
            assert abs(lse[0, t, h] - torch.logsumexp(s, 0).item()) < 1e-12


@pytest.mark.parametrize("window", [4, 0])
def test_row_lse_reproduces_softmax_rows(window):
    """exp(scale q_hat . k_hat - lse) is the softmax row that attention_probs_row returns (the
    probabilities behind the brute-force-pinned prefill oracle), on every row and head."""
    q, k, _, _, _ = _case(6, 1, 12, 8, 2, 16, False)
    kw = dict(rot_dim=6, rope_base=1e4, eps=1e-6)
    lse = oracle.row_lse(q, k, window=window, **kw)
    kh = oracle.qk_prologue(k[0], np.arange(12), None, **kw)
    for t in range(12):
        lo = max(0, t - window + 1) if window > 0 else 0
        qh = oracle.qk_prologue(q[0, t], t, None, **kw)
        p = oracle.attention_probs_row(qh, kh[lo:t + 1], 0.25)               # [Hq, n]
        for h in range(8):
            s = 0.25 * kh[lo:t + 1, h // 4] @ qh[h]
            np.testing.assert_allclose(np.exp(s - lse[0, t, h]), p[h], rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("window,gated", [(0, False), (3, True), (5, False), (0, True)])
def test_backward_rows_match_whole_sequence(window, gated):
    """The row-sampled backward (used at the full bench size, where the whole-sequence form is too
    slow) equals the whole-sequence one (pinned above by finite differences) on every row, and its
    log-sum-exp equals row_lse."""
    B, T, Hq, Hkv, D = 2, 11, 4, 2, 16
    q, k, v, g, dy = _case(40 + window, B, T, Hq, Hkv, D, gated)
    kw = dict(window=window, gated=gated, rot_dim=6, rope_base=100.0, eps=1e-6, pos0=2)
    dq, dk, dv, dg = oracle.layer_backward(q, k, v, g, dy, **kw)
    lse = oracle.row_lse(q, k, window=window, rot_dim=6, rope_base=100.0, eps=1e-6, pos0=2)
    rows_q, rows_k = [0, 3, 4, 10], [0, 1, 6, 9, 10]
    for b in range(B):
        rq, rk, rv, rg, rl = oracle.layer_backward_rows(
            q[b], k[b], v[b], None if g is None else g[b], dy[b], q_rows=rows_q, k_rows=rows_k, **kw)
        np.testing.assert_allclose(rq, dq[b, rows_q], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(rk, dk[b, rows_k], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(rv, dv[b, rows_k], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(rl, lse[b, rows_q], rtol=1e-12, atol=1e-12)
        if gated:
            np.testing.assert_allclose(rg, dg[b, rows_q], rtol=1e-10, atol=1e-12)
