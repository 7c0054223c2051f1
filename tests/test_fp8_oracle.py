"""Pins of the oracle's E4M3 rounding and of decode over an E4M3 KV cache (oracle/fp8.py).

E4M3: OCP 8-bit floats, 4 exponent bits (bias 7), 3 mantissa bits, no infinities, largest finite 448
(the forward-pass format of the pages' FP8 training: ZGCM-1 zh-TW translation page, §3.1)."""
import numpy as np
import pytest
import torch

import oracle
from oracle.fp8 import E4M3_MAX


def test_value_set_from_the_field_definition():
    v = oracle.e4m3_values()
    assert len(v) == 127                      # 0, 7 subnormals, 14 full binades, 7 in the top one
    assert v[0] == 0.0 and v[1] == 2.0 ** -9 and v[-1] == E4M3_MAX
    assert np.all(np.diff(v) > 0)
    assert 2.0 ** -6 in v and 1.0 in v and 240.0 in v and 256.0 in v and 480.0 not in v


def test_every_value_is_a_fixed_point():
    v = oracle.e4m3_values()
    both = np.concatenate([v, -v])
    assert np.array_equal(oracle.round_e4m3(both), both)


def test_midpoints_round_to_even_mantissa():
    v = oracle.e4m3_values()
    mids = (v[:-1] + v[1:]) / 2
    r = oracle.round_e4m3(mids)
    for lo, hi, got in zip(v[:-1], v[1:], r):
        # the neighbour with the even mantissa field: position in the value list is even
        idx_lo = np.searchsorted(v, lo)
        want = lo if idx_lo % 2 == 0 else hi
        assert got == want, (lo, hi, got)
    assert oracle.round_e4m3(1.0625) == 1.0 and oracle.round_e4m3(1.1875) == 1.25
    assert oracle.round_e4m3(17.0) == 16.0 and oracle.round_e4m3(2.0 ** -10) == 0.0


def test_saturation_and_error_bound():
    assert oracle.round_e4m3(460.0) == 448.0 and oracle.round_e4m3(1e6) == 448.0
    assert oracle.round_e4m3(-1e6) == -448.0
    rng = np.random.default_rng(0)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-12, 8, 20000))
    x = x[np.abs(x) <= 440]
    r = oracle.round_e4m3(x)
    v = oracle.e4m3_values()
    idx = np.clip(np.searchsorted(v, np.abs(r)), 1, len(v) - 1)
    spacing = np.maximum(v[idx] - v[idx - 1], v[np.minimum(idx + 1, len(v) - 1)] - v[idx])
    assert np.all(np.abs(r - x) <= spacing / 2 + 1e-300)


def test_matches_torch_float8_e4m3fn_cast():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(100000) * np.exp2(rng.integers(-14, 9, 100000))
    x = x[np.abs(x) < 464]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_e4m3(x), ref)


def _decode_case(seed, R, lens, gated):
    """Caches of E4M3 values; new keys are +-1 patterns (RMSNorm keeps them at +-1 up to eps, and
    RoPE is off), new values are E4M3 values of magnitude >= 2^-4, so rounding the new row to E4M3
    (at scale 1 or 2) only removes the eps."""
    rng = np.random.default_rng(seed)
    B = len(lens)
    codes = lambda *s: oracle.round_e4m3(rng.standard_normal(s))
    kc, vc = codes(B, R, 8, 128), codes(B, R, 8, 128)
    q = rng.standard_normal((B, 32, 128))
    kn = rng.choice([-1.0, 1.0], (B, 8, 128))
    vn = oracle.round_e4m3(rng.choice([-1.0, 1.0], (B, 8, 128)) * rng.uniform(2 ** -4, 8, (B, 8, 128)))
    g = rng.standard_normal((B, 32, 128)) if gated else None
    return kc, vc, q, kn, vn, g, np.array(lens)


@pytest.mark.parametrize("window,R,lens", [(16, 16, [5, 40]), (0, 50, [1, 33])])
def test_decode_over_e4m3_cache(window, R, lens):
    kc, vc, q, kn, vn, g, seq = _decode_case(3, R, lens, gated=window > 0)
    kw = dict(window=window, gated=window > 0, rot_dim=0, rope_base=1e4)
    o1, k1, v1 = oracle.decode_fp8_cache(q, kn, vn, g, kc, vc, seq, k_scale=1.0, v_scale=1.0, **kw)
    # the written row is the rounded k_hat / v
    for b, L in enumerate(seq):
        row = (L - 1) % window if window else L - 1
        khat = oracle.qk_prologue(kn[b], L - 1, None, rot_dim=0, rope_base=1e4, eps=1e-6)
        assert np.array_equal(k1[b, row], oracle.round_e4m3(khat)) and np.all(np.abs(k1[b, row]) == 1)
        assert np.array_equal(v1[b, row], vn[b])
    # halving every stored value and doubling the scales describes the same cache
    o2, k2, v2 = oracle.decode_fp8_cache(q, kn, vn, g, kc / 2, vc / 2, seq, k_scale=2.0,
                                         v_scale=2.0, **kw)
    assert np.allclose(o1, o2, rtol=0, atol=1e-12)
    assert np.array_equal(k2 * 2, k1) and np.array_equal(v2 * 2, v1)
    # the attention is decode() over the same values (which keeps k_hat unrounded: eps apart)
    o3, _, _ = oracle.decode(q, kn, vn, g, kc, vc, seq, **kw)
    assert np.allclose(o1, o3, rtol=0, atol=1e-5)
