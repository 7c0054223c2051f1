"""The Python binding rejects tensors whose shapes disagree with the layer configuration before
anything reaches the library (the C ABI addresses caches and rows from cfg and the sizes it is
given: a ring cache with fewer than `window` rows, say, would otherwise take writes past its end).
Every case raises ValueError on host tensors; no kernel runs."""
import pytest
import torch

import global_causal_attention_amd as zg

bf = torch.bfloat16
RING = zg.AttnConfig(window=128, gated=True)
LIN = zg.AttnConfig(window=0, gated=False)


def _decode_args(B=4, W=128, rows=None, Hq=32, Hkv=8):
    rows = W if rows is None else rows
    return dict(q_new=torch.zeros(B, Hq, 128, dtype=bf), k_new=torch.zeros(B, Hkv, 128, dtype=bf),
                v_new=torch.zeros(B, Hkv, 128, dtype=bf), gate=torch.zeros(B, Hq, 128, dtype=bf),
                k_cache=torch.zeros(B, rows, Hkv, 128, dtype=bf),
                v_cache=torch.zeros(B, rows, Hkv, 128, dtype=bf),
                seqlens=torch.ones(B, dtype=torch.int32))


def _call_decode(cfg, a, max_seqlen=128, fp8=False):
    fn = zg.zg_attn_decode_fp8 if fp8 else zg.zg_attn_decode
    return fn(cfg, a["q_new"], a["k_new"], a["v_new"], a["gate"], a["k_cache"], a["v_cache"],
              a["seqlens"], max_seqlen=max_seqlen)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("field,shape,match", [
    ("k_cache", (4, 64, 8, 128), "k_cache"),       # ring shorter than the window
    ("v_cache", (4, 128, 4, 128), "v_cache"),      # wrong KV head count
    ("q_new", (4, 16, 128), "q_new"),              # wrong query head count
    ("k_new", (4, 8, 64), "k_new"),
    ("v_new", (3, 8, 128), "v_new"),               # batch mismatch
    ("gate", (4, 32, 127), "gate"),
])
def test_decode_rejects_shapes(fp8, field, shape, match):
    a = _decode_args()
    a[field] = torch.zeros(shape, dtype=bf)
    with pytest.raises(ValueError, match=match):
        _call_decode(RING, a, fp8=fp8)


def test_decode_rejects_seqlens_and_short_linear_cache():
    a = _decode_args()
    a["seqlens"] = torch.ones(5, dtype=torch.int32)
    with pytest.raises(ValueError, match="seqlens"):
        _call_decode(RING, a)
    a = _decode_args(rows=100)
    with pytest.raises(ValueError, match="max_seqlen"):
        _call_decode(LIN, a, max_seqlen=200)


def _layer_tensors(B=2, T=10, Hq=32, Hkv=8):
    return (torch.zeros(B, T, Hq, 128, dtype=bf), torch.zeros(B, T, Hkv, 128, dtype=bf),
            torch.zeros(B, T, Hkv, 128, dtype=bf), torch.zeros(B, T, Hq, 128, dtype=bf))


@pytest.mark.parametrize("which,shape", [(0, (2, 10, 16, 128)), (1, (2, 10, 4, 128)),
                                         (2, (2, 9, 8, 128)), (3, (2, 10, 32, 64))])
def test_prefill_rejects_shapes(which, shape):
    t = list(_layer_tensors())
    t[which] = torch.zeros(shape, dtype=bf)
    with pytest.raises(ValueError, match="expected"):
        zg.zg_attn_prefill(RING, *t)
    with pytest.raises(ValueError, match="expected"):
        zg.zg_attn_forward_train(RING, *t)


def test_prefill_rejects_norm_weight_shape():
    with pytest.raises(ValueError, match="q_norm_w"):
        zg.zg_attn_prefill(RING, *_layer_tensors(), q_norm_w=torch.ones(64))


@pytest.mark.parametrize("cfg,rows,match", [(RING, 127, "k_cache"), (LIN, 15, "pos0")])
def test_prefill_cached_rejects_caches(cfg, rows, match):
    q, k, v, g = _layer_tensors()
    kc = torch.zeros(2, rows, 8, 128, dtype=bf)
    with pytest.raises(ValueError, match=match):
        zg.zg_attn_prefill_cached(cfg, q, k, v, g, kc, kc.clone(), pos0=6)


def test_stack_wrappers_reject_shapes():
    x = torch.zeros(1, 4, 4096)
    w_qkvg = torch.zeros((32 + 16 + 32) * 128, 4096, dtype=bf)
    w_o = torch.zeros(4096, 4096, dtype=bf)
    with pytest.raises(ValueError, match="w_qkvg"):
        zg.zg_attn_layer(RING, x, w_qkvg[:-128], w_o)
    with pytest.raises(ValueError, match="w_o"):
        zg.zg_attn_layer(RING, x, w_qkvg, w_o[:, :4000])
    with pytest.raises(ValueError, match="w"):
        zg.zg_gemm_bf16(torch.zeros(8, 256, dtype=bf), torch.zeros(16, 128, dtype=bf))
    with pytest.raises(ValueError, match="residual"):
        zg.zg_gemm_bf16(torch.zeros(8, 128, dtype=bf), torch.zeros(16, 128, dtype=bf),
                        residual=torch.zeros(8, 15))
    with pytest.raises(ValueError, match="w"):
        zg.zg_rmsnorm(torch.zeros(3, 64), w=torch.ones(32))


def test_fp8_stack_wrappers_reject_shapes():
    u8, f32 = torch.uint8, torch.float32
    with pytest.raises(ValueError, match="x_scale"):
        zg.zg_gemm_fp8(torch.zeros(8, 256, dtype=u8), torch.zeros(7, dtype=f32),
                       torch.zeros(16, 256, dtype=u8), torch.zeros(16, dtype=f32))
    with pytest.raises(ValueError, match="w has shape"):
        zg.zg_gemm_fp8(torch.zeros(8, 256, dtype=u8), torch.zeros(8, dtype=f32),
                       torch.zeros(16, 128, dtype=u8), torch.zeros(16, dtype=f32))
    with pytest.raises(ValueError, match="scale"):
        zg.zg_quant_rows_fp8(torch.zeros(4, 64, dtype=bf), scale=torch.zeros(5, dtype=f32))
    x = torch.zeros(1, 4, 4096)
    n_qkvg = (32 + 16 + 32) * 128
    good = dict(w_qkvg=torch.zeros(n_qkvg, 4096, dtype=u8), s_qkvg=torch.zeros(n_qkvg, dtype=f32),
                w_o=torch.zeros(4096, 4096, dtype=u8), s_o=torch.zeros(4096, dtype=f32))
    for name, bad in (("w_qkvg", torch.zeros(n_qkvg - 128, 4096, dtype=u8)),
                      ("s_qkvg", torch.zeros(n_qkvg - 1, dtype=f32)),
                      ("s_o", torch.zeros(4095, dtype=f32))):
        args = dict(good, **{name: bad})
        with pytest.raises(ValueError, match=name):
            zg.zg_attn_layer_fp8(RING, x, args["w_qkvg"], args["s_qkvg"], args["w_o"], args["s_o"])
