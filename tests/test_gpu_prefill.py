"""GPU prefill vs the fp64 oracle on seeded inputs, through the C ABI.

Sizes are small enough for the oracle to finish in seconds but span several query/key tiles and a
ragged tail; the T=1024 gated local layer (seed 1000, base 1e4) is compared in full."""
import numpy as np
import pytest
import torch

import global_causal_attention_amd as zg
import oracle
import synth_inputs as si
from helpers import assert_parity, f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(B, T, Hq, Hkv, W, gated, base, seed, pos0=0, rot=42, norm_w=False, scale=0.0,
         q_scale=1.0):
    print(f"[case] B={B} T={T} Hq={Hq} Hkv={Hkv} W={W} gated={gated} base={base} seed={seed} "
          f"pos0={pos0} rot={rot} norm_w={norm_w}", flush=True)
    gen = si.generator(seed)
    x = si.prefill_layer(gen, B, T, Hq, Hkv, 128, gated=True)
    qw = kw = None
    if norm_w:
        qw = (torch.rand(128, generator=gen) * 1.5 + 0.25) * q_scale
        kw = torch.rand(128, generator=gen) * 1.5 + 0.25
    cfg = zg.AttnConfig(n_q_heads=Hq, n_kv_heads=Hkv, window=W, gated=gated, rot_dim=rot,
                        rope_base=base, softmax_scale=scale)
    dev = {k: (v.to(DEV) if v is not None else None) for k, v in x.items()}
    out = zg.zg_attn_prefill(cfg, dev["q"], dev["k"], dev["v"], dev["gate"],
                             q_norm_w=None if qw is None else qw.to(DEV),
                             k_norm_w=None if kw is None else kw.to(DEV), pos0=pos0)
    torch.cuda.synchronize()
    ref = oracle.prefill(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["gate"]), window=W,
                         gated=gated, rot_dim=rot, rope_base=base, eps=1e-6,
                         q_norm_w=None if qw is None else qw.double().numpy(),
                         k_norm_w=None if kw is None else kw.double().numpy(),
                         scale=scale if scale > 0 else None, pos0=pos0)
    return out, ref


def test_local_layer_T1024_full():
    out, ref = _run(1, 1024, 32, 8, 128, True, 1e4, 1000)
    assert_parity(out, ref, "gated SWA B=1 T=1024")


@pytest.mark.parametrize("B,T,Hq,Hkv,W,gated,base,pos0", [
    (1, 1, 32, 8, 128, True, 1e4, 0),
    (1, 5, 32, 8, 128, True, 1e4, 0),
    (2, 127, 32, 8, 128, True, 1e4, 0),
    (1, 128, 32, 8, 128, True, 1e6, 0),
    (1, 129, 32, 8, 128, True, 1e6, 0),
    (3, 300, 32, 8, 128, True, 1e7, 0),
    (1, 333, 32, 8, 0, False, 1e6, 0),
    (2, 200, 32, 8, 0, True, 1e4, 0),
    (1, 257, 4, 1, 128, True, 1e4, 0),
    (1, 190, 8, 2, 3, True, 1e4, 0),
    (1, 150, 8, 8, 1, False, 1e4, 0),
    (1, 260, 16, 2, 64, True, 1e4, 0),
    (2, 100, 8, 1, 0, False, 1e4, 0),
    (1, 300, 32, 8, 128, True, 1e7, 200000),
    (1, 70, 32, 8, 0, False, 1e7, 262000),
    # four heads per KV head and window <= 128: runs of several 64-query steps per workgroup,
    # run boundaries and ragged tails
    (16, 520, 32, 8, 128, True, 1e4, 0),
    (1, 4100, 32, 8, 128, True, 1e6, 0),
    (1, 1000, 32, 8, 100, False, 1e4, 0),
    (2, 700, 32, 8, 33, True, 1e4, 0),
    (1, 640, 32, 8, 64, True, 1e4, 5),
    (1, 333, 32, 8, 1, True, 1e4, 0),
])
def test_prefill_edges(B, T, Hq, Hkv, W, gated, base, pos0):
    out, ref = _run(B, T, Hq, Hkv, W, gated, base, 7 + T + W, pos0=pos0)
    assert_parity(out, ref, f"B={B} T={T} Hq={Hq}/{Hkv} W={W}")


@pytest.mark.parametrize("B,T,gated,base,pos0,norm_w", [
    # full causal layers with at least two query tiles per compute unit: one workgroup per CU
    # walks the tiles, heavy ones first, bringing the next tile's q rows and first key tiles in
    # while the current one runs (tiles of 1, 2 and >= 3 key tiles mixed, ragged tails)
    (8, 601, True, 1e6, 0, False),
    (16, 300, False, 1e4, 0, True),
    (4, 1030, True, 1e6, 3, False),
    # one and two (sequence, KV head) pairs per XCD: each XCD's light queue holds the light
    # quarter of one or two pairs' tiles, and the launch ends on tiles taken from other XCDs'
    # light queues
    (1, 4160, False, 1e6, 0, False),
    (2, 2100, True, 1e6, 0, False),
])
def test_prefill_persistent_causal(B, T, gated, base, pos0, norm_w):
    out, ref = _run(B, T, 32, 8, 0, gated, base, 17 + T, pos0=pos0, norm_w=norm_w)
    assert_parity(out, ref, f"persistent causal B={B} T={T} gated={gated} norm_w={norm_w}")


@pytest.mark.parametrize("W", [128, 0])
def test_prefill_token_strided_views(W):
    # q, k, v and gate as column slices of one fused [B, T, (2 Hq + 2 Hkv) * 128] projection buffer,
    # out written into a wider buffer
    B, T, Hq, Hkv = 2, 333, 32, 8
    print(f"[case] strided views B={B} T={T} W={W}", flush=True)
    x = si.prefill_layer(si.generator(31 + W), B, T, Hq, Hkv, 128, gated=True)
    fused = torch.cat([x["q"], x["k"], x["v"], x["gate"]], dim=2).to(DEV)
    q, k, v, g = torch.split(fused, [Hq, Hkv, Hkv, Hq], dim=2)
    wide = torch.zeros(B, T, Hq + 3, 128, dtype=torch.bfloat16, device=DEV)
    cfg = zg.AttnConfig(window=W, gated=W > 0, rope_base=1e4)
    zg.zg_attn_prefill(cfg, q, k, v, g if W > 0 else None, out=wide[:, :, :Hq])
    torch.cuda.synchronize()
    ref = oracle.prefill(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["gate"]), window=W,
                         gated=W > 0, rope_base=1e4)
    assert_parity(wide[:, :, :Hq], ref, f"strided views W={W}")
    assert torch.count_nonzero(wide[:, :, Hq:]).item() == 0, "write outside the out view"


def test_prefill_norm_weights_scale_and_rot_dims():
    # rot 42 with non-unit weights runs the banded kernel's folded path (local layer) and the
    # general kernel (causal layer) at normal logit scale
    for W, rot, scale in ((128, 42, 0.0), (0, 42, 0.0), (100, 42, 0.07)):
        out, ref = _run(1, 333, 32, 8, W, W > 0, 1e4, 13 + W, rot=rot, norm_w=True, scale=scale)
        assert_parity(out, ref, f"W={W} rot={rot} scale={scale} with norm weights")
    for rot, scale in ((0, 0.0), (64, 0.05), (16, 0.0)):
        out, ref = _run(1, 200, 32, 8, 128, True, 1e4, 11, rot=rot, norm_w=True, scale=scale)
        assert_parity(out, ref, f"rot={rot} scale={scale} with norm weights")


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).double().numpy()


def _rounded_operand_reference(x, W, gated, qw, kw, base=1e4, folded=False):
    """Test-side model of the kernel's rounding points built on the oracle's prologue; scores are
    in log2 units, the softmax weights are rounded to bf16 and both the weighted sum and the
    normaliser use the rounded weights; everything else is fp64.

    Unfolded (full causal kernel): the matrix cores see bf16(q_hat * scale * log2 e) and
    bf16(k_hat). Folded (banded kernel for 42 rotary dims): they see q with its first 42 dims
    replaced by bf16(RoPE(w_q * q)), and bf16(k_hat * scale * log2 e) with the q norm weight of
    dims >= 42 folded in; the RMS factor of q multiplies the scores."""
    q, k, v = f64(x["q"])[0], f64(x["k"])[0], f64(x["v"])[0]
    T = q.shape[0]
    c = np.log2(np.e) / np.sqrt(128)
    pos = np.arange(T)
    qp = oracle.qk_prologue(q, pos, qw, rot_dim=42, rope_base=base, eps=1e-6)
    kp = oracle.qk_prologue(k, pos, kw, rot_dim=42, rope_base=base, eps=1e-6)
    if folded:
        inv = 1.0 / np.sqrt(np.mean(q * q, axis=-1) + 1e-6)          # [T, Hq]
        qh = q.copy()
        qh[..., :42] = _bf16((qp / inv[..., None])[..., :42])
        fold = np.full(128, c)
        fold[42:] *= qw[42:]
        kh = _bf16(kp * fold)
    else:
        inv = np.ones(q.shape[:2])
        qh = _bf16(c * qp)
        kh = _bf16(kp)
    out = np.zeros(q.shape)
    for t in range(T):
        lo = max(0, t - W + 1) if W > 0 else 0
        s2 = inv[t][:, None] * np.einsum("hd,jhd->hj", qh[t], np.repeat(kh[lo:t + 1], 4, axis=1))
        p = _bf16(np.exp2(s2 - s2.max(-1, keepdims=True)))
        o = np.einsum("hj,jhd->hd", p, np.repeat(v[lo:t + 1], 4, axis=1)) / p.sum(-1)[:, None]
        if gated:
            o = o / (1 + np.exp(-f64(x["gate"])[0, t]))
        out[t] = o
    return out[None]


@pytest.mark.parametrize("W", [0, 128])
def test_prefill_peaky_logits(W):
    """q norm weight ~8 makes logits ~N(0, 64) and exercises the running-max rescale.

    At logit std 8 the bf16 rounding of the matrix-core operands alone moves outputs by up to
    ~0.14 (a test-side emulation of exactly those rounding points reproduces the GPU's error), so
    the fp64-oracle bar is scaled with the logit std: max-abs 2e-2 * 8, mean-abs 2e-3 * 3. The
    tighter check is against the rounding model. The model still differs from the kernel in two
    ways that also scale with the logit std: the kernel's fp32 prologue can round an element of
    q_hat/k_hat to the neighbouring bf16 value of the fp64 one, and the kernel rounds softmax
    weights taken relative to a running reference rather than the final maximum; hence max-abs
    4e-2 there with the standard mean-abs bar."""
    gated = W > 0
    out, ref = _run(1, 400, 32, 8, W, gated, 1e4, 12 + W, norm_w=True, q_scale=8.0)
    assert_parity(out, ref, f"peaky logits W={W} vs fp64 oracle", max_abs=0.16, mean_abs=6e-3)
    gen = si.generator(12 + W)
    x = si.prefill_layer(gen, 1, 400, 32, 8, 128, gated=True)
    qw = ((torch.rand(128, generator=gen) * 1.5 + 0.25) * 8.0).double().numpy()
    kw = (torch.rand(128, generator=gen) * 1.5 + 0.25).double().numpy()
    model = _rounded_operand_reference(x, W, gated, qw, kw, folded=W > 0)
    assert_parity(out, model, f"peaky logits W={W} vs bf16-operand model", max_abs=4e-2)


@pytest.mark.parametrize("W", [0, 128])
def test_prefill_rescale_path_standard_bar(W):
    """The running softmax reference raised many times, held to the bf16 output bar (2e-2 max,
    2e-3 mean) against the fp64 oracle. synth_inputs.ramped_logits_layer sweeps each query's scores
    over about +-90 log2 units (q norm weight 4): in the causal layer every row's first key tile
    has its maximum outside [-32, 32], so the reference is set from it, and about half the rows
    later see scores more than 64 above it; in the banded layer the sawtooth makes the newest
    keys of a window exceed the first block's maximum by more than 60 on about a third of the
    rows. The score differences that decide the weights come from the smooth ramp and v is
    smooth along the keys, so the bf16 rounding of the matrix-core operands moves the output
    little (a CPU model of exactly those rounding points stays within 1.0e-2 / 6.8e-4), while a
    wrong rescale of the running sum or output moves it by O(1)."""
    T = 600
    print(f"[case] rescale path W={W} T={T}", flush=True)
    x = si.ramped_logits_layer(si.generator(4100 + W), T, window=W)
    qw = torch.full((128,), 4.0)
    cfg = zg.AttnConfig(window=W, gated=W > 0, rope_base=1e4)
    dev = {k: v.to(DEV) for k, v in x.items()}
    out = zg.zg_attn_prefill(cfg, dev["q"], dev["k"], dev["v"], dev["gate"] if W else None,
                             q_norm_w=qw.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.prefill(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["gate"]), window=W,
                         gated=W > 0, rope_base=1e4, q_norm_w=qw.double().numpy())
    assert_parity(out, ref, f"rescale path W={W}")
