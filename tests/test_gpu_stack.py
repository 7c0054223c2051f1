"""GPU parity of the attention-only stack pieces (RMSNorm, bf16 GEMM, one whole layer, 32 layers)
against the fp64 oracle, through the C ABI.

Projections follow ZGCM-1 zh-TW translation page §2.1 / Fig. 3 (q, k, v and gate projections of a
normalised hidden state, o_proj after the gated attention; Pre-LN residual). Weights are seeded
N(0, 0.02) bf16 of the real hidden size 4096; sequence lengths are reduced so the fp64 oracle
finishes in seconds, with ragged row counts so tiles are partly filled."""
import numpy as np
import pytest
import torch

import global_causal_attention_amd as zg
import oracle
import synth_inputs as si
import stack_model
from helpers import assert_parity, err_stats, f64

pytestmark = pytest.mark.gpu
DEV = "cuda"
H = 4096


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("rows,dim", [(1, 4096), (301, 4096), (77, 1024)])
def test_rmsnorm(rows, dim):
    print(f"[case] rmsnorm rows={rows} dim={dim}", flush=True)
    g = torch.Generator().manual_seed(rows)
    x = (torch.randn(rows, dim, generator=g) * 3).to(DEV)
    w = (torch.rand(dim, generator=g) + 0.5).to(DEV)
    for wt in (None, w):
        y = zg.zg_rmsnorm(x, 1e-6, wt)
        torch.cuda.synchronize()
        xd = f64(x)
        ref = xd / np.sqrt(np.mean(xd * xd, -1, keepdims=True) + 1e-6)
        if wt is not None:
            ref = ref * f64(wt)
        # one bf16 rounding of an fp32 value: within one bf16 ulp of the fp64 value
        err = np.abs(f64(y) - ref) / np.maximum(np.abs(ref), 1e-30)
        assert err.max() <= 2.0 ** -7, f"rmsnorm rel err {err.max():.3e}"


@pytest.mark.parametrize("M,N,K", [(1, 1024, 4096), (300, 5120, 4096), (129, 4096, 4096),
                                   (64, 200, 128)])
def test_gemm_bf16(M, N, K):
    print(f"[case] gemm M={M} N={N} K={K}", flush=True)
    g = torch.Generator().manual_seed(M + N)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(DEV)
    w = (torch.randn(N, K, generator=g) * 0.02).to(torch.bfloat16).to(DEV)
    r0 = torch.randn(M, N, generator=g).to(DEV)
    res = r0.clone()
    y = zg.zg_gemm_bf16(x, w, residual=res)
    torch.cuda.synchronize()
    ref = f64(x) @ f64(w).T
    # fp32 accumulation of K bf16 products: error far below the bf16 rounding of y
    assert_parity(y, ref, f"gemm y M={M} N={N} K={K}")
    assert np.abs(f64(y) - _bf16(ref)).max() <= 2.0 ** -7 * np.abs(ref).max() + 1e-6
    assert_parity(res, f64(r0) + ref, f"gemm residual M={M} N={N} K={K}", max_abs=1e-3,
                  mean_abs=1e-4)


def _layer_weights(gen, is_global):
    w = si.stack_layer_weights(gen, H, 32, 8, 128, is_global=is_global, device=DEV)
    parts = [w["wq"], w["wk"], w["wv"]] + ([] if is_global else [w["wg"]])
    return w, torch.cat(parts, 0).contiguous()


def _oracle_weights(w):
    return {k: f64(v) for k, v in w.items()}


@pytest.mark.parametrize("is_global,B,T", [(False, 1, 300), (True, 1, 300), (False, 2, 130)])
def test_attn_layer_teacher_forced(is_global, B, T):
    print(f"[case] layer global={is_global} B={B} T={T}", flush=True)
    gen = si.generator(1004 + T + is_global, device=DEV)
    x = si.stack_input(gen, B, T, H, device=DEV)
    w, wqkvg = _layer_weights(gen, is_global)
    cfg = zg.AttnConfig(window=0 if is_global else 128, gated=not is_global, rope_base=1e7)
    x_in = f64(x)
    zg.zg_attn_layer(cfg, x, wqkvg, w["wo"])
    torch.cuda.synchronize()
    ref = oracle.stack_layer(x_in, _oracle_weights(w), is_global=is_global, rope_base=1e7)
    # compare the layer's contribution (the residual stream itself is carried exactly in fp32)
    assert_parity(f64(x) - x_in, ref - x_in, f"layer delta global={is_global} B={B} T={T}")


def test_stack_32_layers_end_to_end():
    """All 32 layers (globals at 6, 12, 18, 24, 30) at T=160 through zg_attn_layer (T > 128, so the
    local layers run the banded kernel on a ragged last step), weights drawn layer by layer so only
    one layer is resident.

    Three checks, with bars fixed before the run from a CPU simulation (an fp32 implementation with
    the GPU's bf16 rounding points, against tests/stack_model.py, at this T):
      1. Every layer on the GPU's own input (teacher forcing): its increment against the rounding
         model's increment, at the bf16 output bar (2e-2 max, 2e-3 mean; the simulation differs
         from the model by 1.0e-3 / 1.4e-5 there). Against the fp64 oracle the increment may
         differ by what the rounding points themselves cause: the bar there is the model's own
         distance from fp64 (max x 1.5, mean x 1.25), since the deep global layers' increments
         (RMS ~1.4) carry a mean rounding error of ~2.0e-3 by themselves.
      2. Free running, layers 1-2: the GPU's residual stream against the rounding model run on its
         own, at the bf16 output bar (simulation: 5.7e-3 / 4.2e-4 at layer 2). Beyond a few layers
         no implementation tracks the model element by element: the bf16 rounding of
         h = RMSNorm(x) turns fp32-level differences in x into whole-ulp differences in h, and the
         simulation drifts from the model by 0.11 max / 0.015 mean at layer 32.
      3. Free running, layer 32: the GPU's distance from the fp64 oracle is no more than the
         rounding model's own (max x 1.5, mean x 1.25; the simulation's ratios are 0.99 and 0.98).
         A wiring mistake (schedule, residual, gate) moves the output by O(1) relative to itself."""
    B, T = 1, 160
    print(f"[case] 32-layer stack B={B} T={T}", flush=True)
    gen = si.generator(1004, device=DEV)
    x = si.stack_input(gen, B, T, H, device=DEV)
    xr = f64(x)[0]          # fp64 oracle, free running
    xm = xr.copy()          # rounding model, free running
    for l in range(1, 33):
        is_global = oracle.layer_is_global(l)
        w, wqkvg = _layer_weights(gen, is_global)
        wh = _oracle_weights(w)
        cfg = zg.AttnConfig(window=0 if is_global else 128, gated=not is_global, rope_base=1e7)
        x_in = f64(x)[0]
        zg.zg_attn_layer(cfg, x, wqkvg, w["wo"])
        torch.cuda.synchronize()
        d_gpu = f64(x)[0] - x_in
        d_mod = stack_model.layer(x_in, wh, is_global=is_global) - x_in
        d_ref = oracle.stack_layer(x_in[None], wh, is_global=is_global, rope_base=1e7)[0] - x_in
        assert_parity(d_gpu, d_mod, f"layer {l} increment vs rounding model (teacher-forced)")
        m_max, m_mean, _ = err_stats(d_mod, d_ref)
        assert_parity(d_gpu, d_ref, f"layer {l} increment vs fp64 (teacher-forced)",
                      max_abs=1.5 * m_max, mean_abs=1.25 * m_mean)
        xr = oracle.stack_layer(xr[None], wh, is_global=is_global, rope_base=1e7)[0]
        xm = stack_model.layer(xm, wh, is_global=is_global)
        if l <= 2:
            assert_parity(f64(x)[0], xm, f"free-running layers 1..{l} vs rounding model")
        del w, wqkvg, wh
    m_max, m_mean, m_rel = err_stats(xm, xr)
    print(f"[parity] rounding model vs fp64 after 32 layers: max_abs={m_max:.3e} "
          f"mean_abs={m_mean:.3e} rel_rms={m_rel:.3e}", flush=True)
    assert_parity(x[0], xr, "32-layer stack output vs fp64", max_abs=1.5 * m_max,
                  mean_abs=1.25 * m_mean)
