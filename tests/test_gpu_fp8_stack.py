"""GPU parity of the E4M3 projections (row quantization, RMSNorm to E4M3, the scaled E4M3 GEMM and a
whole layer with E4M3 projections) against the fp64 oracle, through the C ABI.

The pages train the forward matrix multiplications in FP8 E4M3 (ZGCM-1 zh-TW translation page,
§3.1); the readings (one fp32 scale per row, scale = amax / 448, codes from the fp32 product) are
in oracle/fp8_stack.py and the library header. Bars:

* Quantization of bf16 rows: bit for bit (both sides round the same fp32 product to E4M3).
* RMSNorm to E4M3: the kernel's h is fp32, the oracle's fp64 rounded to fp32; they may differ in the
  last bit, so a code may differ where the product sits on a rounding midpoint: at most 1 in 10^4
  codes differ, each to the adjacent code, with the oracle's product within 2^-20 of the midpoint.
* GEMM: the E4M3 products are exact; the matrix cores sum each 64-product block at reduced precision
  (measured: relative RMS error 5.1e-5 at every K from 128 to 4096, far below the bf16 output's
  2^-9), so the fp32 residual path is held to relative RMS 2e-4 and max 1e-3 of the largest output,
  the bf16 path to one bf16 rounding. Small-integer operands, whose sums fit in 13 bits, are exact.
* Layer: E4M3 quantization turns bf16-level differences upstream (the kernels' bf16 q/k/v, gate and
  attention output against the oracle's fp64 ones) into whole-code flips (2^-3 against 2^-9), so
  two correct implementations of the layer differ by a fraction of what the quantization itself
  moves it. The bar, against the distance between that oracle and the same layer with bf16
  projections: the increment's distance from the fp64 E4M3 oracle at most half of it in mean
  (measured 0.27 to 0.28 at T=130..300) and at most all of it in max (a tail statistic over ~10^6
  elements: measured 0.25 to 0.53); a wiring mistake (a scale, a row, a transposed weight) moves
  the increment by O(1) of itself."""
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


def _values(codes):
    return oracle.e4m3_decode(codes.cpu().numpy())


def _random_codes(g, shape):
    c = torch.randint(0, 255, shape, generator=g, dtype=torch.uint8)
    c[c == 0x7F] = 0          # no NaN codes (0xFF is excluded by the range)
    return c


@pytest.mark.parametrize("rows,dim,strided", [(64, 4096, False), (33, 1024, True), (5, 16, False)])
def test_quant_rows_bit_exact(rows, dim, strided):
    print(f"[case] quant_rows rows={rows} dim={dim} strided={strided}", flush=True)
    g = torch.Generator().manual_seed(rows + dim)
    x = torch.randn(rows, dim, generator=g) * torch.exp2(torch.randint(-12, 12, (rows, 1), generator=g).float())
    x[1] = 0.0                     # a zero row
    x[2] = 0.0
    x[2, dim // 3] = -2.5          # one nonzero element
    xb = x.to(torch.bfloat16)
    if strided:                    # rows of a wider buffer
        wide = torch.zeros(rows, dim + 24, dtype=torch.bfloat16)
        wide[:, 8:8 + dim] = xb
        xd = wide.to(DEV)[:, 8:8 + dim]
    else:
        xd = xb.to(DEV)
    codes, scale = zg.zg_quant_rows_fp8(xd)
    torch.cuda.synchronize()
    vr, sr = oracle.quant_rows_e4m3(xb.float().numpy())
    assert np.array_equal(_values(codes), vr), "codes differ from the oracle's"
    assert np.array_equal(scale.cpu().numpy(), sr), "scales differ from the oracle's"


@pytest.mark.parametrize("rows,dim", [(1, 4096), (301, 4096), (77, 1024)])
def test_rmsnorm_fp8(rows, dim):
    print(f"[case] rmsnorm_fp8 rows={rows} dim={dim}", flush=True)
    g = torch.Generator().manual_seed(7 * rows + dim)
    x = torch.randn(rows, dim, generator=g) * 3
    w = torch.rand(dim, generator=g) + 0.5
    for wt in (None, w):
        codes, scale = zg.zg_rmsnorm_fp8(x.to(DEV), 1e-6, None if wt is None else wt.to(DEV))
        torch.cuda.synchronize()
        xd = x.double().numpy()
        h = xd / np.sqrt(np.mean(xd * xd, -1, keepdims=True) + 1e-6)
        if wt is not None:
            h = h * wt.double().numpy()
        h32 = h.astype(np.float32)
        vr, sr = oracle.quant_rows_e4m3(h32)
        vg = _values(codes)
        sg = scale.cpu().numpy()
        assert np.all(np.abs(sg / sr - 1.0) <= 2.0 ** -22), "scales differ by more than 2 ulp"
        diff = vg != vr
        assert diff.mean() <= 1e-4, f"{diff.sum()} codes differ"
        if diff.any():
            inv = (np.float32(448.0) / np.max(np.abs(h32), axis=1)).astype(np.float64)
            prod = h32.astype(np.float64) * inv[:, None]
            mid = (vg + vr) / 2
            assert np.all(np.abs(prod - mid)[diff] <= 2.0 ** -20 * np.abs(mid)[diff])
            assert np.all(np.abs(vg - vr)[diff] <= np.abs(mid)[diff] * 2.0 ** -2), "not adjacent"


@pytest.mark.parametrize("K,vals", [(128, (0.0, 1.0, -1.0)), (4096, (0.0, 1.0, -1.0)),
                                    (1024, (0.0, 1.0, -1.0, 2.0, -2.0))])
def test_gemm_fp8_small_integers_exact(K, vals):
    """Operands whose sums fit in 13 bits: every output is exact, which pins the operand layout
    (which k each register byte stands for on both sides) and the scale application."""
    print(f"[case] gemm_fp8 exact K={K} vals={vals}", flush=True)
    g = torch.Generator().manual_seed(K)
    M, N = 300, 520
    table = {0.0: 0x00, 1.0: 0x38, -1.0: 0xB8, 2.0: 0x40, -2.0: 0xC0}
    pick = torch.tensor([table[v] for v in vals], dtype=torch.uint8)
    xc = pick[torch.randint(0, len(vals), (M, K), generator=g)]
    wc = pick[torch.randint(0, len(vals), (N, K), generator=g)]
    xs = torch.exp2(torch.randint(-3, 3, (M,), generator=g).float())
    ws = torch.exp2(torch.randint(-3, 3, (N,), generator=g).float())
    res = torch.zeros(M, N, device=DEV)
    zg.zg_gemm_fp8(xc.to(DEV), xs.to(DEV), wc.to(DEV), ws.to(DEV), residual=res, want_y=False)
    torch.cuda.synchronize()
    ref = oracle.gemm_e4m3(_values(xc), xs.numpy(), _values(wc), ws.numpy())
    assert np.array_equal(res.cpu().double().numpy(), ref), "small-integer GEMM not exact"


@pytest.mark.parametrize("M,N,K", [(1, 1024, 4096), (300, 5120, 4096), (129, 4096, 4096),
                                   (64, 200, 128)])
def test_gemm_fp8(M, N, K):
    print(f"[case] gemm_fp8 M={M} N={N} K={K}", flush=True)
    g = torch.Generator().manual_seed(M + N + K)
    xc, wc = _random_codes(g, (M, K)), _random_codes(g, (N, K))
    xs = torch.rand(M, generator=g) * 0.01 + 0.001
    ws = torch.rand(N, generator=g) * 0.01 + 0.001
    r0 = torch.randn(M, N, generator=g)
    res = r0.to(DEV)
    y = zg.zg_gemm_fp8(xc.to(DEV), xs.to(DEV), wc.to(DEV), ws.to(DEV), residual=res)
    torch.cuda.synchronize()
    ref = oracle.gemm_e4m3(_values(xc), xs.numpy(), _values(wc), ws.numpy())
    big = np.abs(ref).max()
    mx, mean, rel = err_stats(f64(res) - r0.double().numpy(), ref)
    print(f"[parity] gemm_fp8 residual M={M} N={N} K={K}: max_abs={mx:.3e} rel_rms={rel:.3e}",
          flush=True)
    assert rel <= 2e-4 and mx <= 1e-3 * big, "residual path beyond the accumulation bar"
    yd = f64(y)
    assert np.abs(yd - stack_model.bf16(ref)).max() <= 2.0 ** -7 * big + 1e-6, "bf16 path"


def test_gemm_fp8_bench_shapes_sampled_rows():
    """The stack's projection shapes at T=65536 (M=65536, K=4096; N=10240 into bf16, N=4096 onto
    an fp32 residual), the whole product on the GPU, 96 rows against the oracle."""
    print("[case] gemm_fp8 M=65536 sampled", flush=True)
    g = torch.Generator(device=DEV).manual_seed(1004)
    M, K = 65536, 4096
    xc = torch.randint(0, 127, (M, K), generator=g, dtype=torch.uint8, device=DEV)
    xc = torch.where(torch.rand(M, K, generator=g, device=DEV) < 0.5, xc, xc | 0x80)
    xs = torch.rand(M, generator=g, device=DEV) * 1e-3 + 1e-4
    rows = np.unique(np.concatenate([[0, 1, 255, 256, M - 2, M - 1],
                                     np.random.default_rng(3).integers(0, M, 90)]))
    for N, resid in ((10240, False), (4096, True)):
        wc = torch.randint(0, 127, (N, K), generator=g, dtype=torch.uint8, device=DEV)
        wc = torch.where(torch.rand(N, K, generator=g, device=DEV) < 0.5, wc, wc | 0x80)
        ws = torch.rand(N, generator=g, device=DEV) * 1e-3 + 1e-4
        res = torch.zeros(M, N, device=DEV) if resid else None
        y = zg.zg_gemm_fp8(xc, xs, wc, ws, residual=res, want_y=not resid)
        torch.cuda.synchronize()
        out = f64((res if resid else y)[torch.from_numpy(rows).to(DEV)])
        ref = oracle.gemm_e4m3(_values(xc[torch.from_numpy(rows).to(DEV)]), xs.cpu().numpy()[rows],
                               _values(wc), ws.cpu().numpy())
        big = np.abs(ref).max()
        mx, mean, rel = err_stats(out, ref)
        print(f"[parity] gemm_fp8 N={N} sampled rows: max_abs={mx:.3e} rel_rms={rel:.3e}", flush=True)
        if resid:
            assert rel <= 2e-4 and mx <= 1e-3 * big
        else:
            assert np.abs(out - stack_model.bf16(ref)).max() <= 2.0 ** -7 * big + 1e-6
        del res, y, wc


@pytest.mark.parametrize("is_global,B,T", [(False, 1, 300), (True, 1, 300), (False, 2, 130)])
def test_attn_layer_fp8_teacher_forced(is_global, B, T):
    print(f"[case] fp8 layer global={is_global} B={B} T={T}", flush=True)
    gen = si.generator(1004 + T + is_global, device=DEV)
    x = si.stack_input(gen, B, T, H, device=DEV)
    w = si.stack_layer_weights(gen, H, 32, 8, 128, is_global=is_global, device=DEV)
    names = ["wq", "wk", "wv"] + ([] if is_global else ["wg"])
    wqkvg = torch.cat([w[n] for n in names], 0).contiguous()
    cq, sq = zg.zg_quant_rows_fp8(wqkvg)
    co, so = zg.zg_quant_rows_fp8(w["wo"])
    cfg = zg.AttnConfig(window=0 if is_global else 128, gated=not is_global, rope_base=1e7)
    x_in = f64(x)
    zg.zg_attn_layer_fp8(cfg, x, cq, sq, co, so)
    torch.cuda.synchronize()
    wf = oracle.quantize_layer_weights({n: f64(t) for n, t in w.items()})
    # the library's weight codes and scales are the oracle's
    assert np.array_equal(_values(cq), np.concatenate([wf[n][0] for n in names], 0))
    assert np.array_equal(sq.cpu().numpy(), np.concatenate([wf[n][1] for n in names], 0))
    assert np.array_equal(_values(co), wf["wo"][0])
    d_gpu = f64(x) - x_in
    d_ref = oracle.stack_layer_fp8(x_in, wf, is_global=is_global, rope_base=1e7) - x_in
    d16 = oracle.stack_layer(x_in, {n: f64(t) for n, t in w.items()}, is_global=is_global,
                             rope_base=1e7) - x_in
    q_max, q_mean, q_rel = err_stats(d_ref, d16)   # what E4M3 projections change in the oracle
    print(f"[fp8] E4M3 vs bf16 projections (oracle): max_abs={q_max:.3e} mean_abs={q_mean:.3e} "
          f"rel_rms={q_rel:.3e}", flush=True)
    assert_parity(d_gpu, d_ref, f"fp8 layer increment vs fp64 E4M3 oracle global={is_global}",
                  max_abs=q_max, mean_abs=0.5 * q_mean)
    # and the GPU's layer is the quantized one: far closer to the E4M3 oracle than to bf16
    assert err_stats(d_gpu, d_ref)[2] < 0.5 * err_stats(d_gpu, d16)[2]
