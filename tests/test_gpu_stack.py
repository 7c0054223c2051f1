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
from helpers import assert_parity, f64

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
    """All 32 layers (globals at 6, 12, 18, 24, 30) at T=96, GPU and oracle each carrying their
    own residual stream; weights are drawn layer by layer so only one layer is resident.

    Bar: the output is the fp32 residual after 32 layers (RMS ~5 here), not a bf16 tensor, so the
    bf16 output bar does not apply to it directly. Each layer contributes with a relative error of
    ~5e-3 (its bf16 operands: the teacher-forced test above holds it to the bf16 bar), and the
    errors compound through the later layers' norms; the check is relative RMS error <= 1e-2 and
    max-abs error <= 2e-2 of the output's largest magnitude. Any wiring mistake (layer schedule,
    residual, gate) moves the output by O(1) relative to itself."""
    B, T = 1, 96
    print(f"[case] 32-layer stack B={B} T={T}", flush=True)
    gen = si.generator(1004, device=DEV)
    x = si.stack_input(gen, B, T, H, device=DEV)
    xr = f64(x)
    for l in range(1, 33):
        is_global = oracle.layer_is_global(l)
        w, wqkvg = _layer_weights(gen, is_global)
        cfg = zg.AttnConfig(window=0 if is_global else 128, gated=not is_global, rope_base=1e7)
        zg.zg_attn_layer(cfg, x, wqkvg, w["wo"])
        xr = oracle.stack_layer(xr, _oracle_weights(w), is_global=is_global, rope_base=1e7)
        del w, wqkvg
    torch.cuda.synchronize()
    scale = float(np.abs(xr).max())
    mx, mean, rel = assert_parity(x, xr, "32-layer stack output", max_abs=2e-2 * scale,
                                  mean_abs=np.inf)
    assert rel <= 1e-2, f"32-layer stack: relative RMS error {rel:.3e} > 1e-2"
