"""zg_attn_decode_noalloc (the decode step with the library's static per-device scratch instead of
a caller workspace, for callers that cannot allocate) against zg_attn_decode on the same inputs,
through the C ABI: two calls in a row, the second with a smaller batch and shorter contexts, so the
second reads a scratch the first left full of its own partials. Outputs and cache writes must be
bit-identical to the workspace entry point's (the same kernels on the same inputs), and within the
bf16 output bar of the fp64 oracle on a few sequences."""
import numpy as np
import pytest
import torch

import global_causal_attention_amd as zg
import oracle
import synth_inputs as si
from helpers import assert_parity, f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _step(seed, B, lo, hi, window):
    x = si.decode_step(si.generator(seed, device=DEV), B=B, len_lo=lo, len_hi=hi, device=DEV)
    cfg = zg.AttnConfig(window=window, gated=window > 0, rope_base=1e7)
    kc, vc = (x["ring_k"], x["ring_v"]) if window else (x["lin_k"], x["lin_v"])
    g = x["gate"] if window else None
    # the workspace entry point on copies of the caches
    kc_a, vc_a = kc.clone(), vc.clone()
    ref = zg.zg_attn_decode(cfg, x["q_new"], x["k_new"], x["v_new"], g, kc_a, vc_a, x["seqlens"],
                            max_seqlen=hi)
    kc_b, vc_b = kc.clone(), vc.clone()
    got = zg.zg_attn_decode_noalloc(cfg, x["q_new"], x["k_new"], x["v_new"], g, kc_b, vc_b,
                                    x["seqlens"], max_seqlen=hi)
    torch.cuda.synchronize()
    assert_parity(got, f64(ref), f"noalloc vs workspace decode B={B} W={window}")
    assert torch.equal(got, ref), "noalloc decode differs from the workspace entry point"
    assert torch.equal(kc_a, kc_b) and torch.equal(vc_a, vc_b), "cache writes differ"
    seq = x["seqlens"].cpu().numpy()
    for b in (0, B - 1):
        L = int(seq[b])
        rows = slice(None) if window else slice(0, L)
        r, _, _ = oracle.decode(f64(x["q_new"][b:b + 1]), f64(x["k_new"][b:b + 1]),
                                f64(x["v_new"][b:b + 1]), None if g is None else f64(g[b:b + 1]),
                                f64(kc[b:b + 1, rows]), f64(vc[b:b + 1, rows]), seq[b:b + 1],
                                window=window, gated=window > 0, rope_base=1e7)
        assert_parity(got[b:b + 1], r, f"noalloc decode sequence {b} (L={L}) vs oracle")


def test_noalloc_decode_two_calls():
    print("[case] noalloc decode: B=64 L~U[8192,65536] linear, then B=8 L~U[1000,3000] linear, "
          "then B=16 rings", flush=True)
    _step(5001, 64, 8192, 65536, 0)      # 64 chunks per sequence: the partials fill ~67 MB
    _step(5002, 8, 1000, 3000, 0)        # smaller: reads a scratch left full by the first call
    _step(5003, 16, 200, 3000, 128)      # rings (one chunk per sequence)


def test_noalloc_decode_rejects_oversize():
    x = si.decode_step(si.generator(5004, device=DEV), B=2, len_lo=10, len_hi=20, device=DEV)
    cfg = zg.AttnConfig(window=0, gated=False, rope_base=1e7)
    big = 1 << 21
    kc = torch.zeros(2, 1, 8, 128, dtype=torch.bfloat16, device=DEV).expand(2, big, 8, 128)
    with pytest.raises((zg.ZGError, ValueError)):
        zg.zg_attn_decode_noalloc(cfg, x["q_new"], x["k_new"], x["v_new"], None, kc, kc,
                                  x["seqlens"], max_seqlen=big)
