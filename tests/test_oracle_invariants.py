"""Properties the mathematics fixes, checked on the fp64 oracle (no GPU)."""
import numpy as np
import pytest
import torch

import oracle


def _inputs(seed, B=1, T=40, Hq=8, Hkv=2, D=16):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, T, Hq, D)), rng.standard_normal((B, T, Hkv, D)),
            rng.standard_normal((B, T, Hkv, D)), rng.standard_normal((B, T, Hq, D)))


KW = dict(rot_dim=6, rope_base=1e4, eps=1e-6)


@pytest.mark.parametrize("T", [1, 5, 17])
def test_window_at_least_T_equals_full_causal(T):
    q, k, v, g = _inputs(1, T=T)
    full = oracle.prefill(q, k, v, g, window=0, gated=True, **KW)
    for W in (T, T + 1, 128):
        band = oracle.prefill(q, k, v, g, window=W, gated=True, **KW)
        assert np.array_equal(band, full)


def test_zero_gate_is_exactly_half():
    q, k, v, _ = _inputs(2)
    ungated = oracle.prefill(q, k, v, None, window=8, gated=False, **KW)
    zero = np.zeros(q.shape)
    gated = oracle.prefill(q, k, v, zero, window=8, gated=True, **KW)
    assert np.array_equal(gated, 0.5 * ungated)


def test_probabilities_sum_to_one_and_v_one_gives_one():
    q, k, v, _ = _inputs(3)
    qhat = oracle.qk_prologue(q[0, 30], 30, None, **KW)
    khat = oracle.qk_prologue(k[0, 10:31], np.arange(10, 31), None, **KW)
    p = oracle.attention_probs_row(qhat, khat, 0.25)
    assert p.shape == (8, 21)
    assert np.all(p > 0)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-14)
    ones = np.ones_like(v)
    out = oracle.prefill(q, k, ones, None, window=7, gated=False, **KW)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-14)


def test_rope_preserves_pair_norms_and_passthrough():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((50, 3, 128))
    pos = rng.integers(0, 262144, 50)
    y = oracle.partial_rope(x, pos, 42, 1e7)
    n_in = x[..., :21] ** 2 + x[..., 21:42] ** 2
    n_out = y[..., :21] ** 2 + y[..., 21:42] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=1e-13, atol=1e-13)
    assert np.array_equal(y[..., 42:], x[..., 42:])
    # position 0 is the identity
    assert np.array_equal(oracle.partial_rope(x, np.zeros(50, int), 42, 1e7), x)


def test_rope_equals_complex_rotation_and_composes():
    """RoPE pair (i, i+half) is multiplication by exp(i*pos*theta_i) in the complex plane, so
    rotating by p then by r equals rotating by p + r."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 2, 128))
    half = 21
    theta = 1e6 ** (-np.arange(half) / half)
    for p in (0, 1, 1000, 262143):
        y = oracle.partial_rope(x, np.full(4, p), 42, 1e6)
        z = (x[..., :half] + 1j * x[..., half:42]) * np.exp(1j * p * theta)
        np.testing.assert_allclose(y[..., :half], z.real, atol=1e-12)
        np.testing.assert_allclose(y[..., half:42], z.imag, atol=1e-12)
    a = oracle.partial_rope(oracle.partial_rope(x, np.full(4, 300), 42, 1e6), np.full(4, 77), 42, 1e6)
    b = oracle.partial_rope(x, np.full(4, 377), 42, 1e6)
    np.testing.assert_allclose(a, b, atol=1e-10)


def test_shift_invariance_of_outputs():
    """Scores depend only on relative positions, so moving every position by c leaves the output."""
    q, k, v, g = _inputs(6, T=24, D=32)
    kw = dict(rot_dim=12, rope_base=1e4, eps=1e-6)
    a = oracle.prefill(q, k, v, g, window=5, gated=True, pos0=0, **kw)
    b = oracle.prefill(q, k, v, g, window=5, gated=True, pos0=12345, **kw)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-9)


def test_rmsnorm_mean_square_identity_and_torch():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((20, 128)) * rng.uniform(0.01, 30, (20, 1))
    eps = 1e-6
    y = oracle.rms_norm(x, None, eps)
    ms = np.mean(x * x, -1)
    np.testing.assert_allclose(np.mean(y * y, -1), ms / (ms + eps), rtol=1e-13)
    w = rng.uniform(0.5, 2, 128)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(w), eps)
    np.testing.assert_allclose(oracle.rms_norm(x, w, eps), ref.numpy(), rtol=1e-13, atol=1e-13)


def test_single_key_closed_forms():
    q, k, v, g = _inputs(8, T=12)
    sig = 1.0 / (1.0 + np.exp(-g))
    out = oracle.prefill(q, k, v, g, window=0, gated=True, **KW)
    # query 0 sees only key 0: o = v_0 * sigmoid(g)
    G = 4
    np.testing.assert_allclose(out[0, 0], np.repeat(v[0, 0], G, axis=0) * sig[0, 0], atol=1e-14)
    # window 1: every query sees only itself
    out1 = oracle.prefill(q, k, v, g, window=1, gated=True, **KW)
    np.testing.assert_allclose(out1[0], np.repeat(v[0], G, axis=1) * sig[0], atol=1e-14)


def test_uniform_keys_give_window_mean():
    """Keys equal at every position with zero rotated dims: all scores tie, so o is the mean of v
    over the key set."""
    q, _, v, _ = _inputs(9, T=30)
    k = np.zeros((1, 30, 2, 16))
    k[..., 6:] = np.random.default_rng(10).standard_normal(10)
    out = oracle.prefill(q, k, v, None, window=7, gated=False, **KW)
    for t in range(30):
        lo = max(0, t - 6)
        mean = v[0, lo:t + 1].mean(0)                      # [Hkv, D]
        np.testing.assert_allclose(out[0, t], np.repeat(mean, 4, axis=0), atol=1e-13)


def test_ring_slot_permutation_invariance():
    rng = np.random.default_rng(11)
    B, Hq, Hkv, D, W = 2, 8, 2, 16, 8
    kc = rng.standard_normal((B, W, Hkv, D))
    vc = rng.standard_normal((B, W, Hkv, D))
    qn, gn = rng.standard_normal((B, Hq, D)), rng.standard_normal((B, Hq, D))
    kn, vn = rng.standard_normal((B, Hkv, D)), rng.standard_normal((B, Hkv, D))
    seqlens = np.array([50, 70])
    a, ka, va = oracle.decode(qn, kn, vn, gn, kc, vc, seqlens, window=W, gated=True, **KW)
    # Relabel which slot holds which cached entry (keeping the new token's slot): same output.
    perm = np.arange(W)
    for b in range(B):
        s_new = (seqlens[b] - 1) % W
        others = [s for s in range(W) if s != s_new]
        perm_b = perm.copy()
        perm_b[others] = np.array(others)[::-1]
        kc2, vc2 = kc.copy(), vc.copy()
        kc2[b] = kc[b, perm_b]
        vc2[b] = vc[b, perm_b]
        b_out, _, _ = oracle.decode(qn, kn, vn, gn, kc2, vc2, seqlens, window=W, gated=True, **KW)
        np.testing.assert_allclose(b_out[b], a[b], atol=1e-13)
    # the new key lands in slot pos % W
    for b in range(B):
        s = (seqlens[b] - 1) % W
        np.testing.assert_allclose(va[b, s], vn[b])
        np.testing.assert_allclose(ka[b, s], oracle.qk_prologue(kn[b], seqlens[b] - 1, None, **KW))


def test_decode_linear_ignores_rows_beyond_position():
    rng = np.random.default_rng(12)
    B, Hq, Hkv, D, R = 1, 4, 1, 8, 20
    kc = rng.standard_normal((B, R, Hkv, D))
    vc = rng.standard_normal((B, R, Hkv, D))
    args = [rng.standard_normal((B, Hq, D)), rng.standard_normal((B, Hkv, D)),
            rng.standard_normal((B, Hkv, D)), None]
    a, _, _ = oracle.decode(*args, kc, vc, np.array([9]), window=0, gated=False, **KW)
    kc[:, 9:] = 1e6
    vc[:, 9:] = -1e6
    b, _, _ = oracle.decode(*args, kc, vc, np.array([9]), window=0, gated=False, **KW)
    np.testing.assert_array_equal(a, b)
