"""Pins of the stack oracle (Pre-LN attention-only layers with projections)."""
import numpy as np
import pytest

import oracle

SMALL = dict(n_q_heads=4, n_kv_heads=1, head_dim=8, window=4, rot_dim=2, rope_base=1e4, eps=1e-6)
H = 32  # hidden = n_q_heads * head_dim


def _weights(rng, is_global, scale=0.3):
    w = {"wq": rng.standard_normal((32, H)) * scale, "wk": rng.standard_normal((8, H)) * scale,
         "wv": rng.standard_normal((8, H)) * scale, "wo": rng.standard_normal((H, 32)) * scale}
    if not is_global:
        w["wg"] = rng.standard_normal((32, H)) * scale
    return w


def test_zero_output_projection_keeps_residual():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((2, 9, H))
    w = _weights(rng, False)
    w["wo"][:] = 0
    np.testing.assert_array_equal(oracle.stack_layer(x, w, is_global=False, **SMALL), x)


def test_single_token_closed_form():
    """T = 1: one key, so attention returns v; the layer adds (v * sigmoid(g)) @ Wo^T, with
    h = x / rms(x), v = h Wv^T repeated over the 4 query heads of the group."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((1, 1, H))
    for is_global in (False, True):
        w = _weights(rng, is_global)
        h = x[0, 0] / np.sqrt(np.mean(x[0, 0] ** 2) + 1e-6)
        v = h @ w["wv"].T                                   # [8] = one kv head
        a = np.tile(v, 4)                                    # 4 query heads share it
        if not is_global:
            a = a / (1 + np.exp(-(h @ w["wg"].T)))
        expect = x[0, 0] + a @ w["wo"].T
        got = oracle.stack_layer(x, w, is_global=is_global, **SMALL)
        np.testing.assert_allclose(got[0, 0], expect, atol=1e-12)


def test_zero_gate_weights_halve_local_increment():
    """For T <= window local and global key sets coincide; with W_g = 0 the gate is sigmoid(0) =
    1/2, so a local layer adds exactly half of what the same layer adds as a global layer."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1, 4, H))
    w = _weights(rng, False)
    w["wg"][:] = 0
    loc = oracle.stack_layer(x, w, is_global=False, **SMALL) - x
    glo = oracle.stack_layer(x, w, is_global=True, **SMALL) - x
    np.testing.assert_allclose(loc, 0.5 * glo, atol=1e-14)


def test_stack_applies_schedule():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 6, H))
    ws = [_weights(rng, oracle.layer_is_global(l, 3)) for l in range(1, 7)]
    y = oracle.stack(x, ws, global_every=3, **SMALL)
    z = x
    for l, w in enumerate(ws, 1):
        z = oracle.stack_layer(z, w, is_global=(l % 3 == 0), **SMALL)
    np.testing.assert_array_equal(y, z)
    assert [l for l in range(1, 33) if oracle.layer_is_global(l)] == [6, 12, 18, 24, 30]


def test_rows_form_equals_whole_layer():
    """stack_layer_rows (projections only where the requested rows need them) equals stack_layer on
    every row, for both layer types, a window shorter than the sequence, a position offset and an
    unsorted subset of rows."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, 11, H))
    for is_global in (False, True):
        w = _weights(rng, is_global)
        full = oracle.stack_layer(x, w, is_global=is_global, pos0=5, **SMALL)
        for b in range(2):
            got = oracle.stack_layer_rows(x[b], w, range(11), is_global=is_global, pos0=5, **SMALL)
            np.testing.assert_allclose(got, full[b], rtol=0, atol=1e-12)
        got = oracle.stack_layer_rows(x[1], w, [10, 0, 6], is_global=is_global, pos0=5, **SMALL)
        np.testing.assert_allclose(got, full[1][[10, 0, 6]], rtol=0, atol=1e-12)


@pytest.mark.parametrize("is_global", [False, True])
def test_rounding_model_without_rounding_is_the_oracle(is_global, monkeypatch):
    """tests/stack_model.py (the GPU's bf16 rounding points inserted into the oracle's arithmetic)
    reduces to oracle.stack_layer when its rounding is switched off: the folded score form of the
    local layer (RMS factor applied to the scores, reference subtracted) is exact in real
    arithmetic, so a wiring mistake in the model shows here."""
    import stack_model
    monkeypatch.setattr(stack_model, "bf16", lambda a: np.asarray(a, dtype=np.float64))
    rng = np.random.default_rng(5 + is_global)
    T, hidden = 150, 4096
    x = rng.standard_normal((T, hidden))
    w = {n: rng.standard_normal(s) * 0.02 for n, s in
         (("wq", (4096, hidden)), ("wk", (1024, hidden)), ("wv", (1024, hidden)),
          ("wg", (4096, hidden)), ("wo", (hidden, 4096)))}
    got = stack_model.layer(x, w, is_global=is_global, rope_base=1e7)
    ref = oracle.stack_layer(x[None], w, is_global=is_global, rope_base=1e7)[0]
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-10)
