"""GPU parity of decode over E4M3 KV caches (zg_attn_decode_fp8) and of the bf16 -> E4M3 conversion
(zg_kv_to_fp8) against the fp64 oracle (oracle/fp8.py), through the C ABI.

E4M3 is the forward-pass FP8 format of the pages' training (ZGCM-1 zh-TW translation page, §3.1);
the cache holds E4M3 values that stand for value * scale. Cache contents are seeded N(0,1) draws
cast to E4M3 by torch (input generation); both sides attend over exactly those values, so the output
bar is the standard one (max-abs 2e-2, mean-abs 2e-3). The new token's row is rounded on the GPU
from the fp32 k_hat and by the oracle from the fp64 one: a code may differ where k_hat lies within
fp32 rounding of a rounding boundary, so the written keys are checked as a correct rounding of the
oracle's k_hat (within half a spacing, plus 1e-5 relative), and identical in at least 99% of
elements; values are exact (v / scale is exact for the power-of-two scales used)."""
import numpy as np
import pytest
import torch

import global_causal_attention_amd as zg
import oracle
from helpers import assert_parity, f64

pytestmark = pytest.mark.gpu
DEV = "cuda"
D = 128


def _e4m3(gen, shape):
    return torch.randn(shape, generator=gen).to(torch.float8_e4m3fn)


def _spacing(v):
    """E4M3 spacing at |v| (the gap above |v|'s binade start; subnormal spacing below 2^-6)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 2.0 ** (np.minimum(e, 8) - 3)


CASES = [  # Hq, Hkv, window, lens, k_scale, v_scale
    (32, 8, 128, [200, 128, 5, 1000], 1.0, 1.0),
    (32, 8, 64, [64, 65, 300, 1], 0.5, 2.0),      # another ring width, scaled E4M3 entries
    (32, 8, 0, [1, 2048, 3000], 0.5, 2.0),
    (32, 8, 0, [777, 1024, 1025], 1.0, 0.25),
    (32, 4, 0, [1500, 60], 1.0, 1.0),       # 8 query heads per KV head
    (16, 16, 128, [300, 2], 2.0, 1.0),      # one query head per KV head
]


@pytest.mark.parametrize("Hq,Hkv,window,lens,ks,vs", CASES)
def test_decode_fp8(Hq, Hkv, window, lens, ks, vs):
    print(f"[case] fp8 decode Hq={Hq} Hkv={Hkv} W={window} lens={lens} scales={ks},{vs}", flush=True)
    gen = torch.Generator().manual_seed(3000 + window + sum(lens))
    B = len(lens)
    gated = window > 0
    R = window if window else max(lens) + 7
    kc, vc = _e4m3(gen, (B, R, Hkv, D)), _e4m3(gen, (B, R, Hkv, D))
    q = torch.randn(B, Hq, D, generator=gen).to(torch.bfloat16)
    kn = torch.randn(B, Hkv, D, generator=gen).to(torch.bfloat16)
    vn = torch.randn(B, Hkv, D, generator=gen).to(torch.bfloat16)
    g = torch.randn(B, Hq, D, generator=gen).to(torch.bfloat16) if gated else None
    seq = torch.tensor(lens, dtype=torch.int32)
    cfg = zg.AttnConfig(n_q_heads=Hq, n_kv_heads=Hkv, window=window, gated=gated, rope_base=1e7)
    kc_d, vc_d = kc.to(DEV), vc.to(DEV)
    out = zg.zg_attn_decode_fp8(cfg, q.to(DEV), kn.to(DEV), vn.to(DEV),
                                g.to(DEV) if gated else None, kc_d, vc_d, seq.to(DEV),
                                max_seqlen=R if not window else max(lens), k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    ref, rk, rv = oracle.decode_fp8_cache(f64(q), f64(kn), f64(vn), None if g is None else f64(g),
                                          f64(kc), f64(vc), seq.numpy(), k_scale=ks, v_scale=vs,
                                          window=window, gated=gated, rope_base=1e7)
    assert_parity(out, ref, f"fp8 decode W={window} G={Hq // Hkv}")
    got_k, got_v = f64(kc_d), f64(vc_d)
    match, total = 0, 0
    for b, L in enumerate(lens):
        row = (L - 1) % window if window else L - 1
        khat = oracle.qk_prologue(f64(kn)[b], L - 1, None, rot_dim=42, rope_base=1e7, eps=1e-6) / ks
        gk = got_k[b, row]
        assert np.all(np.abs(gk - np.clip(khat, -448, 448)) <= 0.5 * _spacing(gk) + 1e-5 * np.abs(khat)), \
            f"sequence {b}: written key is not a rounding of k_hat"
        match += int(np.sum(gk == rk[b, row]))
        total += gk.size
        assert np.array_equal(got_v[b, row], rv[b, row]), f"sequence {b}: written value"
        # every other row is untouched
        other = np.ones(R, bool)
        other[row] = False
        assert np.array_equal(got_k[b, other], f64(kc)[b, other])
    assert match >= 0.99 * total, f"written key codes agree in {match}/{total}"


def test_kv_to_fp8_matches_oracle_rounding():
    gen = torch.Generator().manual_seed(3100)
    x = (torch.randn(4, 1000, 16, generator=gen) * 40).to(torch.bfloat16)
    x[0, 0, :4] = torch.tensor([1000.0, -1000.0, 460.0, 2.0 ** -10])
    for scale in (1.0, 0.5, 3.0):
        got = zg.zg_kv_to_fp8(x.to(DEV), scale=scale)
        torch.cuda.synchronize()
        ref = oracle.round_e4m3(f64(x) / np.float32(scale))  # the kernel divides in fp32
        assert np.array_equal(f64(got), ref), f"scale {scale}"
