"""The oracle's attention core against torch's CPU fp64 scaled_dot_product_attention.

Norm and RoPE are made exact identities (eps = 0 and +-1 entries make RMSNorm divide by exactly 1;
rot_dim = 0), and the RMSNorm weight carries arbitrary magnitudes, so q_hat = sign * w exactly. The
library routine then sees an explicit boolean band mask and GQA-repeated keys and values.
"""
import numpy as np
import pytest
import torch

import oracle


@pytest.mark.parametrize("T,W,Hq,Hkv", [(1, 4, 4, 1), (64, 4, 8, 2), (130, 128, 32, 8),
                                        (300, 1, 4, 1), (70, 0, 8, 2), (100, 33, 4, 4)])
def test_core_matches_sdpa(T, W, Hq, Hkv):
    rng = np.random.default_rng(T + W)
    B, D = 2, 16
    qs = rng.choice([-1.0, 1.0], (B, T, Hq, D))
    ks = rng.choice([-1.0, 1.0], (B, T, Hkv, D))
    v = rng.standard_normal((B, T, Hkv, D))
    g = rng.standard_normal((B, T, Hq, D))
    wq = rng.uniform(0.1, 1.5, D)
    wk = rng.uniform(0.1, 1.5, D)
    got = oracle.prefill(qs, ks, v, g, window=W, gated=True, rot_dim=0, rope_base=1e4, eps=0.0,
                         q_norm_w=wq, k_norm_w=wk)
    G = Hq // Hkv
    qt = torch.from_numpy(qs * wq).permute(0, 2, 1, 3)                     # [B,Hq,T,D]
    kt = torch.from_numpy(ks * wk).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    mask = (j <= i) & ((i - j < W) if W > 0 else torch.ones(T, T, dtype=torch.bool))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    ref = ref.permute(0, 2, 1, 3) * torch.sigmoid(torch.from_numpy(g))
    np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-12)
