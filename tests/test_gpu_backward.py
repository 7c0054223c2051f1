"""GPU parity of the training path through the C ABI: zg_attn_forward_train (out and the row
log-sum-exp) and zg_attn_backward (dq, dk, dv, dgate) against the fp64 oracle (oracle.backward:
the chain rule applied step by step to the plain forward definition, pinned by finite differences
in test_backward_oracle.py). ZGCM-1 zh-TW translation page, section 2.1 and Figure 3 (the layer),
sections 2.2 and 3.1 (training throughput).

Bar for the gradients. The GPU rounds q_hat, k_hat, dO, P and dS to bf16 (relative 2^-9) at the
matrix-core inputs and accumulates in fp32, so each gradient carries a relative error of a few
2^-9 per rounded factor; dS = P (dP - D) loses a little more to cancellation. Measured against the
size of each gradient: relative RMS error <= 1e-2 and max-abs error <= 3e-2 * max |ref|
(about 15 ulp of bf16 at the largest element); measured: relative RMS <= 4.8e-3, max <= 8.7e-3.
With one token dq and dk are exactly 0 while the GPU's D = sum(dy * y) uses the bf16-rounded y,
so there they are held to the absolute bar 2e-2. The forward's bf16 output is held to the bf16
output bar (max-abs 2e-2, mean-abs 2e-3), as prefill's is. The row log-sum-exp is compared absolutely:
<= 2e-2, the bf16 rounding of q_hat and k_hat moving a score of size |s| by about |s| 2^-8.
"""
import numpy as np
import pytest
import torch

import global_causal_attention_amd as zg
import oracle
import synth_inputs as si
from helpers import assert_parity, f64

pytestmark = pytest.mark.gpu
DEV = "cuda"
D = 128
REL_RMS = 1e-2
REL_MAX = 3e-2
LSE_ABS = 2e-2

CASES = [  # window, gated, B, T, Hq, Hkv
    (128, True, 1, 300, 32, 8),   # local layer: several tiles and a ragged tail
    (0, False, 2, 200, 32, 8),    # global layer, two sequences
    (64, True, 1, 130, 8, 2),     # another window
    (0, False, 1, 517, 8, 2),     # global, many key tiles
    (0, True, 1, 64, 8, 2),       # one exact tile, gated global
    (128, True, 2, 100, 8, 2),    # window covering the sequence: causal
    (0, True, 1, 1, 8, 2),        # one token
]


def _check(got, ref, what):
    """Errors relative to the gradient's size; a gradient that is exactly 0 (one token: the softmax
    over a single key is constant) is held to the absolute bar 2e-2 instead."""
    g = f64(got)
    e = np.abs(g - ref)
    scale = float(np.abs(ref).max())
    if scale == 0.0:
        print(f"[parity] {what}: exact gradient 0, max_abs={e.max():.3e}", flush=True)
        return float(e.max() / 2e-2 * REL_MAX), 0.0
    rel_rms = float(np.sqrt(np.mean(e ** 2)) / np.sqrt(np.mean(ref ** 2)))
    rel_max = float(e.max() / scale)
    print(f"[parity] {what}: max|ref|={scale:.3e} rel_max={rel_max:.3e} rel_rms={rel_rms:.3e}",
          flush=True)
    return rel_max, rel_rms


@pytest.mark.parametrize("W,gated,B,T,Hq,Hkv", CASES)
def test_backward_matches_oracle(W, gated, B, T, Hq, Hkv):
    print(f"[case] backward W={W} gated={gated} B={B} T={T} Hq={Hq} Hkv={Hkv}", flush=True)
    gen = si.generator(3000 + W + T + Hq)
    x = si.prefill_layer(gen, B, T, Hq, Hkv, D, gated=gated)
    dy = si.randn_bf16(gen, (B, T, Hq, D))
    cfg = zg.AttnConfig(n_q_heads=Hq, n_kv_heads=Hkv, window=W, gated=gated)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    g = x["gate"].to(DEV) if gated else None
    out, lse = zg.zg_attn_forward_train(cfg, q, k, v, g)
    dq, dk, dv, dg = zg.zg_attn_backward(cfg, q, k, v, g, out, dy.to(DEV), lse)
    torch.cuda.synchronize()

    qh, kh, vh, dyh = f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(dy)
    gh = f64(x["gate"]) if gated else None
    ref_out = oracle.prefill(qh, kh, vh, gh, window=W, gated=gated)
    ref_lse = oracle.row_lse(qh, kh, window=W)
    rdq, rdk, rdv, rdg = oracle.layer_backward(qh, kh, vh, gh, dyh, window=W, gated=gated)

    # the forward output is a bf16 output like prefill's: the standard bar
    assert_parity(out, ref_out, f"forward_train out W={W} T={T}")
    res = {}
    lse_err = float(np.abs(f64(lse) - ref_lse).max())
    print(f"[parity] lse: max_abs={lse_err:.3e}", flush=True)
    res["dq"] = _check(dq, rdq, "dq")
    res["dk"] = _check(dk, rdk, "dk")
    res["dv"] = _check(dv, rdv, "dv")
    if gated:
        res["dgate"] = _check(dg, rdg, "dgate")
    assert lse_err <= LSE_ABS, f"lse max abs err {lse_err:.3e}"
    for name, (rel_max, rel_rms) in res.items():
        assert np.isfinite(rel_max), f"{name}: non-finite"
        assert rel_rms <= REL_RMS, f"{name}: relative RMS error {rel_rms:.3e} > {REL_RMS}"
        assert rel_max <= REL_MAX, f"{name}: max error {rel_max:.3e} of max|ref| > {REL_MAX}"


def test_backward_rejects_unsupported_ratio():
    x = si.prefill_layer(si.generator(1), 1, 8, 8, 1, D, gated=False)
    cfg = zg.AttnConfig(n_q_heads=8, n_kv_heads=1, window=0, gated=False)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    with pytest.raises(zg.ZGError):
        zg.zg_attn_forward_train(cfg, q, k, v)


def _sample_rows(gen, T, fixed, n_rand):
    r = torch.randint(0, T, (n_rand,), generator=gen).tolist()
    return sorted(set(int(t) for t in list(fixed) + r if 0 <= t < T))


@pytest.mark.parametrize("layer", ["swa", "global"])
def test_backward_fullsize_sampled(layer):
    """B=4, T=16384 with the inputs and launch configuration of bench.py's training layers (the
    same seed and draw order): the whole backward runs on the GPU; dq, dgate and the log-sum-exp
    are checked on sampled query rows and dk, dv on sampled key rows of the first and last
    sequence, against the row-restricted chain rule (oracle.layer_backward_rows). For the global
    layer the sampled keys sit in the last 64 positions, whose query sets are short enough for the
    oracle; every sampled query row reads its whole prefix."""
    B, T, Hq, Hkv = 4, 16384, 32, 8
    print(f"[case] backward full size {layer} B={B} T={T}", flush=True)
    gen = si.generator(1007, device="cuda")
    for name, win in (("swa", 128), ("global", 0)):  # bench.py's draw order
        x = si.prefill_layer(gen, B, T, Hq, Hkv, D, gated=win > 0, device="cuda")
        dy = si.randn_bf16(gen, (B, T, Hq, D), device="cuda")
        if name == layer:
            break
    W, gated = (128, True) if layer == "swa" else (0, False)
    cfg = zg.AttnConfig(window=W, gated=gated, rope_base=1e6)
    g = x["gate"] if gated else None
    out, lse = zg.zg_attn_forward_train(cfg, x["q"], x["k"], x["v"], g)
    dq, dk, dv, dg = zg.zg_attn_backward(cfg, x["q"], x["k"], x["v"], g, out, dy, lse)
    torch.cuda.synchronize()

    pick = torch.Generator().manual_seed(5)
    got = {n: [] for n in ("dq", "dk", "dv", "dgate", "lse")}
    ref = {n: [] for n in got}
    for b in (0, B - 1):
        q_rows = _sample_rows(pick, T, [0, 1, 63, 64, 127, 128, 2047, 2048, 8191, T - 65, T - 64,
                                        T - 2, T - 1], 4)
        if W:
            k_rows = _sample_rows(pick, T, [0, 63, 64, 4095, T - 129, T - 1], 3)
        else:
            k_rows = [T - 64, T - 63, T - 33, T - 2, T - 1]
        cpu = lambda t: t[b].float().cpu().numpy()
        rq, rk, rv, rg, rl = oracle.layer_backward_rows(
            cpu(x["q"]), cpu(x["k"]), cpu(x["v"]), cpu(g) if gated else None, cpu(dy),
            window=W, gated=gated, q_rows=q_rows, k_rows=k_rows, rope_base=1e6)
        got["dq"].append(f64(dq[b, q_rows])); ref["dq"].append(rq)
        got["dk"].append(f64(dk[b, k_rows])); ref["dk"].append(rk)
        got["dv"].append(f64(dv[b, k_rows])); ref["dv"].append(rv)
        got["lse"].append(f64(lse[b, q_rows])); ref["lse"].append(rl)
        if gated:
            got["dgate"].append(f64(dg[b, q_rows])); ref["dgate"].append(rg)
    lse_err = float(np.abs(np.concatenate(got["lse"]) - np.concatenate(ref["lse"])).max())
    print(f"[parity] lse: max_abs={lse_err:.3e}", flush=True)
    assert lse_err <= LSE_ABS
    for name in ("dq", "dk", "dv", "dgate"):
        if not ref[name]:
            continue
        rel_max, rel_rms = _check(torch.from_numpy(np.concatenate(got[name])),
                                  np.concatenate(ref[name]), name)
        assert rel_rms <= REL_RMS, f"{name}: relative RMS error {rel_rms:.3e}"
        assert rel_max <= REL_MAX, f"{name}: max error {rel_max:.3e} of max|ref|"
