"""Pins of the E4M3 projection oracle (oracle/fp8_stack.py): the code table, per-row quantization,
the scaled E4M3 GEMM and the layer with E4M3 projections.

E4M3 is the forward-pass format of the pages' FP8 training (ZGCM-1 zh-TW translation page, §3.1);
here it carries the layer's projections, each row with one fp32 scale."""
import numpy as np
import torch

import oracle
from oracle.fp8 import E4M3_MAX


def test_decode_every_code_from_the_field_definition():
    codes = np.arange(256)
    v = oracle.e4m3_decode(codes)
    pos = oracle.e4m3_values()
    assert np.array_equal(v[:127], pos)                 # 0x00..0x7E ascend through the value set
    assert np.isnan(v[127]) and np.isnan(v[255])        # 0x7F, 0xFF
    assert np.array_equal(v[128:255], -pos)             # the sign bit
    assert oracle.e4m3_decode(0x38) == 1.0 and oracle.e4m3_decode(0x7E) == E4M3_MAX
    assert oracle.e4m3_decode(0x01) == 2.0 ** -9 and oracle.e4m3_decode(0x08) == 2.0 ** -6


def test_quant_rows_zero_row_and_row_maximum():
    x = np.zeros((3, 64), np.float32)
    x[1, 5] = -3.5
    x[1, 7] = 1.0
    x[2] = np.linspace(-2.0, 7.0, 64, dtype=np.float32)
    v, s = oracle.quant_rows_e4m3(x)
    assert s[0] == 1.0 and np.all(v[0] == 0.0)
    assert v[1, 5] == -E4M3_MAX and s[1] == np.float32(3.5) / np.float32(448.0)
    assert v[2, -1] == E4M3_MAX and np.max(np.abs(v)) == E4M3_MAX


def test_quant_rows_error_bound_and_round_trip():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((200, 128)) * np.exp2(rng.integers(-8, 8, (200, 1)))).astype(np.float32)
    v, s = oracle.quant_rows_e4m3(x)
    inv = (np.float32(448.0) / np.max(np.abs(x), axis=1)).astype(np.float32)
    prod = (x * inv[:, None]).astype(np.float64)
    normal = np.abs(prod) >= 2.0 ** -6
    # half a spacing: 2^-4 relative in the normal range, 2^-10 absolute below it
    assert np.all(np.abs(v - prod)[normal] <= np.abs(prod)[normal] * 2.0 ** -4)
    assert np.all(np.abs(v - prod)[~normal] <= 2.0 ** -10)
    # a row that already is E4M3 values with its maximum at 448 comes back exactly, scale 1
    row = oracle.e4m3_values()[::3].copy()
    row[-1] = E4M3_MAX
    v2, s2 = oracle.quant_rows_e4m3(np.concatenate([row, -row])[None].astype(np.float32))
    assert s2[0] == 1.0 and np.array_equal(v2[0], np.concatenate([row, -row]))


def test_quant_rows_matches_torch_cast_of_the_fp32_products():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((64, 256)) * np.exp2(rng.integers(-10, 10, (64, 1)))).astype(np.float32)
    v, s = oracle.quant_rows_e4m3(x)
    amax = torch.from_numpy(x).abs().amax(dim=1)
    inv = torch.tensor(448.0, dtype=torch.float32) / amax
    prod = torch.from_numpy(x) * inv[:, None]
    ref = prod.to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(v, ref)
    assert np.array_equal(s, (amax / torch.tensor(448.0, dtype=torch.float32)).numpy())


def test_gemm_matches_brute_force():
    rng = np.random.default_rng(5)
    M, N, K = 5, 7, 9
    vals = oracle.e4m3_values()
    xv = rng.choice(vals, (M, K)) * rng.choice([-1.0, 1.0], (M, K))
    wv = rng.choice(vals, (N, K)) * rng.choice([-1.0, 1.0], (N, K))
    xs = rng.uniform(0.01, 2.0, M).astype(np.float32)
    ws = rng.uniform(0.01, 2.0, N).astype(np.float32)
    y = oracle.gemm_e4m3(xv, xs, wv, ws)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += (xv[m, k] * float(xs[m])) * (wv[n, k] * float(ws[n]))
            assert abs(y[m, n] - acc) <= 1e-12 * max(1.0, abs(acc))


def _weights(rng, hidden, Hq, Hkv, D, gated):
    w = {"wq": rng.standard_normal((Hq * D, hidden)) * 0.05,
         "wk": rng.standard_normal((Hkv * D, hidden)) * 0.05,
         "wv": rng.standard_normal((Hkv * D, hidden)) * 0.05,
         "wo": rng.standard_normal((hidden, Hq * D)) * 0.05}
    if gated:
        w["wg"] = rng.standard_normal((Hq * D, hidden)) * 0.05
    # bf16 weights, as the library takes them
    return {n: torch.from_numpy(a).to(torch.bfloat16).double().numpy() for n, a in w.items()}


def test_row_restricted_layer_equals_whole_layer():
    rng = np.random.default_rng(6)
    Hq, Hkv, D, T = 4, 1, 16, 40
    hidden = Hq * D
    x = rng.standard_normal((1, T, hidden))
    for is_global in (False, True):
        wf = oracle.quantize_layer_weights(_weights(rng, hidden, Hq, Hkv, D, not is_global))
        kw = dict(is_global=is_global, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, window=8, rot_dim=6)
        full = oracle.stack_layer_fp8(x, wf, **kw)[0]
        rows = list(range(T))
        part = oracle.stack_layer_rows_fp8(x[0], wf, rows, **kw)
        assert np.allclose(part, full, rtol=0, atol=1e-12)


def test_zero_output_projection_leaves_x():
    rng = np.random.default_rng(7)
    Hq, Hkv, D, T = 4, 1, 16, 12
    hidden = Hq * D
    x = rng.standard_normal((2, T, hidden))
    w = _weights(rng, hidden, Hq, Hkv, D, True)
    w["wo"] = np.zeros_like(w["wo"])
    wf = oracle.quantize_layer_weights(w)
    y = oracle.stack_layer_fp8(x, wf, is_global=False, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D,
                               window=4, rot_dim=6)
    assert np.array_equal(y, x)
