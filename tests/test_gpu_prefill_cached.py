"""GPU parity of chunked prefill through the decode caches (zg_attn_prefill_cached) against the fp64
oracle, through the C ABI: two chunks of each sequence, the caches they leave, and a decode step
that continues from those caches. ZGCM-1 zh-TW translation page, section 2.3 (local layers keep a
fixed 128-token window, global layers the whole sequence).

The oracle runs the plain definition over the whole sequence (prefill rows pos0 .. pos0+T-1 of the
concatenated chunks, then the decode row); the expected cache rows are its normalised, rotated keys
(one bf16 rounding: relative 2^-7) and the values bit for bit.

Ring chunks whose context is 0 or 63 (mod 64) rows run on the banded streaming kernel (context keys
folded as they are gathered, the ring rewritten from unfolded copies): contexts 0, 127, 64 and 63
below (gated and ungated); the partly filled ring of 60 rows takes the general tiled kernel."""
import numpy as np
import pytest
import torch

import global_causal_attention_amd as zg
import oracle
import synth_inputs as si
from helpers import assert_parity, f64

pytestmark = pytest.mark.gpu
DEV = "cuda"
HQ, HKV, D = 32, 8, 128

CASES = [  # window, gated, B, T1, T2, RoPE base
    (128, True, 2, 200, 150, 1e7),   # ring full before chunk 2; chunk 2 longer than the window
    (128, True, 1, 60, 300, 1e6),    # ring partly filled before chunk 2
    (128, True, 2, 130, 64, 1e7),    # chunk 2 shorter than the window: the ring keeps chunk-1 rows
    (128, True, 1, 64, 200, 1e6),    # 64 context rows: key rows offset by a whole tile
    (128, False, 2, 150, 100, 1e6),  # ungated ring layer, 127 context rows
    (64, True, 1, 100, 37, 1e4),     # another window
    (0, False, 2, 200, 150, 1e7),    # linear caches (global layer)
    (0, False, 1, 1, 257, 1e6),      # one-token first chunk
    (0, True, 1, 70, 90, 1e6),       # gated layer on a linear cache
]


def _khat(k_b, base):
    """Oracle k_hat of one sequence's keys at positions 0 .. L-1."""
    return oracle.qk_prologue(k_b, np.arange(k_b.shape[0]), None, rot_dim=42, rope_base=base,
                              eps=1e-6)


@pytest.mark.parametrize("W,gated,B,T1,T2,base", CASES)
def test_two_chunks_then_decode(W, gated, B, T1, T2, base):
    L = T1 + T2
    print(f"[case] cached prefill W={W} gated={gated} B={B} T1={T1} T2={T2} base={base}", flush=True)
    x = si.prefill_layer(si.generator(2000 + W + T1 + T2), B, L + 1, HQ, HKV, D, gated=gated)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    g = x["gate"].to(DEV) if gated else None
    cfg = zg.AttnConfig(window=W, gated=gated, rope_base=base)
    rows = W if W else L + 3
    kc = torch.zeros(B, rows, HKV, D, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    outs = []
    for lo, hi in ((0, T1), (T1, L)):
        c = lambda t: t[:, lo:hi].contiguous()  # the ABI takes [B, T, ...] token-major tensors
        outs.append(zg.zg_attn_prefill_cached(cfg, c(q), c(k), c(v), c(g) if gated else None,
                                              kc, vc, pos0=lo))
    torch.cuda.synchronize()
    qh, kh, vh = f64(x["q"]), f64(x["k"]), f64(x["v"])
    gh = f64(x["gate"]) if gated else None
    ref = oracle.prefill(qh[:, :L], kh[:, :L], vh[:, :L], None if gh is None else gh[:, :L],
                         window=W, gated=gated, rope_base=base)
    assert_parity(torch.cat(outs, 1), ref, f"chunks W={W} T1={T1} T2={T2}")

    # the caches now hold the normalised, rotated keys and the values of the kept positions
    kept = range(max(0, L - W), L) if W else range(L)
    kc_h, vc_h = kc.float().cpu().numpy(), vc.cpu()
    for b in range(B):
        khat = _khat(kh[b, :L], base)
        for p in kept:
            slot = p % W if W else p
            rel = np.abs(kc_h[b, slot] - khat[p]) / np.maximum(np.abs(khat[p]), 1e-6)
            assert rel.max() <= 2.0 ** -7, f"k cache, sequence {b}, position {p}: rel {rel.max():.2e}"
            assert torch.equal(vc_h[b, slot], x["v"][b, p]), f"v cache, sequence {b}, position {p}"

    # decode continues from the caches at position L
    seq = torch.full((B,), L + 1, dtype=torch.int32, device=DEV)
    out_d = zg.zg_attn_decode(cfg, q[:, L].contiguous(), k[:, L].contiguous(), v[:, L].contiguous(),
                              g[:, L].contiguous() if gated else None, kc, vc, seq,
                              max_seqlen=L + 1)
    torch.cuda.synchronize()
    ref_d = oracle.prefill_rows(qh, kh, vh, gh, [L], window=W, gated=gated, rope_base=base)
    assert_parity(out_d, ref_d[:, 0], f"decode after chunks W={W} L={L}")


@pytest.mark.parametrize("weights", [False, True])
def test_first_chunk_equals_plain_prefill(weights):
    """pos0 = 0 through the caches computes the same attention as the plain prefill call; on the
    banded streaming kernel both calls take the same folded keys from the K prologue kernel, so the
    same output bit for bit (also with non-unit q and k norm weights)."""
    B, T = 2, 333
    gen = si.generator(2100 + weights)
    x = si.prefill_layer(gen, B, T, HQ, HKV, D, gated=True)
    q, k, v, g = (x[n].to(DEV) for n in ("q", "k", "v", "gate"))
    nw = {}
    if weights:
        nw = {"q_norm_w": (torch.rand(D, generator=gen) * 1.5 + 0.25).to(DEV),
              "k_norm_w": (torch.rand(D, generator=gen) * 1.5 + 0.25).to(DEV)}
    print(f"[case] pos0=0 cached vs plain weights={weights}", flush=True)
    for W in (128, 0):
        cfg = zg.AttnConfig(window=W, gated=W > 0, rope_base=1e6)
        kc = torch.zeros(B, W if W else T, HKV, D, dtype=torch.bfloat16, device=DEV)
        vc = torch.zeros_like(kc)
        a = zg.zg_attn_prefill_cached(cfg, q, k, v, g if W else None, kc, vc, pos0=0, **nw)
        ref = zg.zg_attn_prefill(cfg, q, k, v, g if W else None, **nw)
        torch.cuda.synchronize()
        assert_parity(a, f64(ref), f"pos0=0 cached vs plain W={W}", max_abs=2e-2, mean_abs=2e-3)
        if W:  # both run the banded streaming kernel on the same folded keys
            assert torch.equal(a, ref), "pos0=0 cached vs plain: banded kernel results differ"



@pytest.mark.parametrize("T1,T2", [(127, 150), (64, 200)])
def test_ring_chunks_with_norm_weights(T1, T2):
    """Ring chunks on the banded streaming kernel (context 127 = 63 mod 64, or 64 = 0 mod 64) with
    non-unit q and k norm weights: the context keys are gathered from the ring with the q weights
    of dims >= 42 folded in, against the whole-sequence oracle with the same weights; the ring
    then holds the unfolded normalised keys, and decode continues with the same weights."""
    W, B, base = 128, 2, 1e6
    L = T1 + T2
    print(f"[case] cached ring with norm weights T1={T1} T2={T2}", flush=True)
    gen = si.generator(2200 + T1)
    x = si.prefill_layer(gen, B, L + 1, HQ, HKV, D, gated=True)
    qw = torch.rand(D, generator=gen) * 1.5 + 0.25
    kw = torch.rand(D, generator=gen) * 1.5 + 0.25
    q, k, v, g = (x[n].to(DEV) for n in ("q", "k", "v", "gate"))
    qwd, kwd = qw.to(DEV), kw.to(DEV)
    cfg = zg.AttnConfig(window=W, gated=True, rope_base=base)
    kc = torch.zeros(B, W, HKV, D, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    outs = []
    for lo, hi in ((0, T1), (T1, L)):
        c = lambda t: t[:, lo:hi].contiguous()
        outs.append(zg.zg_attn_prefill_cached(cfg, c(q), c(k), c(v), c(g), kc, vc, pos0=lo,
                                              q_norm_w=qwd, k_norm_w=kwd))
    torch.cuda.synchronize()
    qh, kh, vh, gh = (f64(x[n]) for n in ("q", "k", "v", "gate"))
    qwh, kwh = qw.double().numpy(), kw.double().numpy()
    ref = oracle.prefill(qh[:, :L], kh[:, :L], vh[:, :L], gh[:, :L], window=W, gated=True,
                         rope_base=base, q_norm_w=qwh, k_norm_w=kwh)
    assert_parity(torch.cat(outs, 1), ref, f"ring chunks with norm weights T1={T1} T2={T2}")
    kc_h = kc.float().cpu().numpy()
    for b in range(B):
        khat = oracle.qk_prologue(kh[b, :L], np.arange(L), kwh, rot_dim=42, rope_base=base,
                                  eps=1e-6)
        for p in range(L - W, L):
            rel = np.abs(kc_h[b, p % W] - khat[p]) / np.maximum(np.abs(khat[p]), 1e-6)
            assert rel.max() <= 2.0 ** -7, f"k cache, sequence {b}, position {p}: rel {rel.max():.2e}"
    seq = torch.full((B,), L + 1, dtype=torch.int32, device=DEV)
    out_d = zg.zg_attn_decode(cfg, q[:, L].contiguous(), k[:, L].contiguous(), v[:, L].contiguous(),
                              g[:, L].contiguous(), kc, vc, seq, max_seqlen=L + 1, q_norm_w=qwd,
                              k_norm_w=kwd)
    torch.cuda.synchronize()
    ref_d = oracle.prefill_rows(qh, kh, vh, gh, [L], window=W, gated=True, rope_base=base,
                                q_norm_w=qwh, k_norm_w=kwh)
    assert_parity(out_d, ref_d[:, 0], f"decode after ring chunks with norm weights L={L}")
