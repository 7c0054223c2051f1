"""GPU decode (ring and linear caches) vs the fp64 oracle through the C ABI."""
import numpy as np
import pytest
import torch

import global_causal_attention_amd as zg
import oracle
import synth_inputs as si
from helpers import assert_parity, f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _decode_case(B, W, lens, seed, Hq=32, Hkv=8, base=1e7, gated=None, stride=None):
    gated = (W > 0) if gated is None else gated
    print(f"[case] decode B={B} W={W} lens={list(lens)[:6]}... seed={seed}", flush=True)
    gen = si.generator(seed)
    seqlens = torch.tensor(lens, dtype=torch.int32)
    rows = W if W > 0 else (stride or int(max(lens)))
    kc = si.randn_bf16(gen, (B, rows, Hkv, 128))
    vc = si.randn_bf16(gen, (B, rows, Hkv, 128))
    qn = si.randn_bf16(gen, (B, Hq, 128))
    kn = si.randn_bf16(gen, (B, Hkv, 128))
    vn = si.randn_bf16(gen, (B, Hkv, 128))
    g = si.randn_bf16(gen, (B, Hq, 128))
    cfg = zg.AttnConfig(n_q_heads=Hq, n_kv_heads=Hkv, window=W, gated=gated, rope_base=base)
    kcd, vcd = kc.to(DEV), vc.to(DEV)
    out = zg.zg_attn_decode(cfg, qn.to(DEV), kn.to(DEV), vn.to(DEV), g.to(DEV), kcd, vcd,
                            seqlens.to(DEV), max_seqlen=int(max(lens)))
    torch.cuda.synchronize()
    ref, kref, vref = oracle.decode(f64(qn), f64(kn), f64(vn), f64(g), f64(kc), f64(vc),
                                    seqlens.numpy(), window=W, gated=gated, rope_base=base)
    return out, ref, kcd, vcd, kref, vref, seqlens


@pytest.mark.parametrize("B,W,lens", [
    (4, 128, [1, 2, 128, 129]),
    (3, 128, [127, 300, 1000]),
    (2, 4, [3, 50]),
    (5, 0, [1, 2, 1023, 1024, 1025]),
    (3, 0, [5000, 2048, 3071]),
])
def test_decode_small(B, W, lens):
    out, ref, kcd, vcd, kref, vref, seqlens = _decode_case(B, W, lens, 100 + B + W)
    assert_parity(out, ref, f"decode W={W}")
    # the new key/value landed in their rows; other rows untouched
    for b in range(B):
        pos = lens[b] - 1
        row = pos % W if W > 0 else pos
        assert_parity(kcd[b, row], kref[b, row], "k_hat written to the cache", max_abs=4e-2,
                      mean_abs=1e-2)
        np.testing.assert_array_equal(f64(vcd[b, row]), vref[b, row])
        other = [r for r in range(kcd.shape[1]) if r != row]
        np.testing.assert_array_equal(f64(kcd[b, other]), kref[b, other])


def test_decode_grouping_variants():
    for Hq, Hkv in ((4, 1), (8, 2), (8, 8), (16, 2)):
        out, ref, *_ = _decode_case(2, 0, [1500, 2600], 200 + Hq, Hq=Hq, Hkv=Hkv, gated=True)
        assert_parity(out, ref, f"decode Hq/Hkv={Hq}/{Hkv}")
