"""GPU parity at the benchmark sizes, on sampled outputs the fp64 oracle computes one by one.

Workloads (seeded N(0,1) bf16, drawn on the device with a seeded generator; the oracle reads the
same tensors copied to the host):
  * B=4, T=16384 gated local layer (W=128) and full causal layer, RoPE base 1e6 (the timed 5:1
    block): sampled query rows of every sequence, all 32 heads, in the launch configuration the
    benchmark times (runs of 32 steps of 64 queries for the local layer);
  * B=64 decode step, 128-slot rings and linear caches with context lengths uniform on
    [8192, 65536], base 1e7: every sequence of both, and every sequence of the same step over the
    linear caches converted to E4M3;
  * B=1, T=262144 gated local and full causal layers, base 1e7: sampled rows (256 seeded uniform
    rows plus the edges for the local layer; a global row at this length costs the fp64 oracle
    about 4.3 GFLOP, so the global layer takes 40);
  * chunked prefill, B=4 sequences with 16384 cached positions continuing with 2048 new tokens,
    base 1e6 (128-slot rings: the banded streaming kernel on a 127-row context; linear caches):
    sampled new rows of the first and last sequence.
Sampled rows cover the sequence edges, tile/step/run boundaries (+-1 around multiples of 32, 64,
128 and 2048) and seeded uniform positions (B=4, T=16384: 512 per layer, the same rows in every
sequence)."""
import numpy as np
import pytest
import torch

import global_causal_attention_amd as zg
import oracle
import synth_inputs as si
from helpers import assert_parity, f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _host(t):
    return t.float().cpu().numpy()


def _rows(T, n_uniform, seed):
    edges = {0, 1, 2, 126, 127, 128, 129, T - 2, T - 1}
    for m in (32, 128):  # +-1 around the first multiples of 32 and 128 and some in the middle
        for c in list(range(m, 8 * m, m)) + [T // 2 + m, T - m]:
            edges |= {c - 1, c, c + 1}
    for m in (64, 2048):
        for c in range(m, T, max(m, T // 8)):
            edges |= {c - 1, c, c + 1}
    rng = np.random.default_rng(seed)
    edges |= set(rng.integers(0, T, n_uniform).tolist())
    return sorted(r for r in edges if 0 <= r < T)


def _layer(B, T, seed, base):
    gen = si.generator(seed, device=DEV)
    return si.prefill_layer(gen, B, T, 32, 8, 128, gated=True, device=DEV)


@pytest.mark.parametrize("W", [128, 0])
def test_b4_t16384_sampled_rows(W):
    B, T, base = 4, 16384, 1e6
    print(f"[case] B={B} T={T} W={W} base={base}", flush=True)
    x = _layer(B, T, 1001, base)
    cfg = zg.AttnConfig(window=W, gated=W > 0, rope_base=base)
    out = zg.zg_attn_prefill(cfg, x["q"], x["k"], x["v"], x["gate"] if W else None)
    torch.cuda.synchronize()
    rows = _rows(T, 512, 11 + W)
    q, k, v, g = (_host(x[n]) for n in ("q", "k", "v", "gate"))
    got = _host(out[:, rows])
    if W:
        ref = np.concatenate([oracle.prefill_rows(q, k, v, g, [r], window=W, gated=True,
                                                  rope_base=base) for r in rows], axis=1)
    else:
        ref = oracle.prefill_rows(q, k, v, None, rows, window=0, gated=False, rope_base=base)
    assert_parity(got, ref, f"B=4 T=16384 W={W}, {len(rows)} rows x 4 sequences")


def test_b64_decode_rings_and_linear_caches():
    Bd, lo, hi = 64, 8192, 65536
    print(f"[case] decode B={Bd} L~U[{lo},{hi}]", flush=True)
    x = si.decode_step(si.generator(1002, device=DEV), B=Bd, len_lo=lo, len_hi=hi, device=DEV)
    seq = x["seqlens"]
    seq_h = seq.cpu().numpy()
    # local layer: 128-slot rings, gated
    cfg = zg.AttnConfig(window=128, gated=True, rope_base=1e7)
    kc, vc = x["ring_k"].clone(), x["ring_v"].clone()
    out = zg.zg_attn_decode(cfg, x["q_new"], x["k_new"], x["v_new"], x["gate"], kc, vc, seq,
                            max_seqlen=hi)
    torch.cuda.synchronize()
    ref, rk, rv = oracle.decode(_host(x["q_new"]), _host(x["k_new"]), _host(x["v_new"]),
                                _host(x["gate"]), _host(x["ring_k"]), _host(x["ring_v"]), seq_h,
                                window=128, gated=True, rope_base=1e7)
    assert_parity(out, ref, "decode B=64 rings")
    rel = np.abs(kc.float().cpu().numpy() - rk) / np.maximum(np.abs(rk), 1e-6)
    assert rel.max() <= 2.0 ** -7, f"ring K after the write: rel {rel.max():.2e}"
    assert torch.equal(vc.cpu(), torch.from_numpy(rv).to(torch.bfloat16)), "ring V write"
    # global layer: linear caches, ungated; every sequence against the oracle, one at a time
    cfg = zg.AttnConfig(window=0, gated=False, rope_base=1e7)
    kc, vc = x["lin_k"], x["lin_v"]
    out = zg.zg_attn_decode(cfg, x["q_new"], x["k_new"], x["v_new"], None, kc, vc, seq,
                            max_seqlen=hi)
    torch.cuda.synchronize()
    for b in range(Bd):
        L = int(seq_h[b])
        r, rk, _ = oracle.decode(_host(x["q_new"][b:b + 1]), _host(x["k_new"][b:b + 1]),
                                 _host(x["v_new"][b:b + 1]), None, _host(kc[b:b + 1, :L]),
                                 _host(vc[b:b + 1, :L]), seq_h[b:b + 1], window=0, gated=False,
                                 rope_base=1e7)
        assert_parity(out[b:b + 1], r, f"decode linear sequence {b} (L={L})")
        # the written row is one bf16 rounding of the fp32 k_hat: within a bf16 ulp of fp64
        got_k, ref_k = kc[b, L - 1].float().cpu().numpy(), rk[0, L - 1]
        rel = np.abs(got_k - ref_k) / np.maximum(np.abs(ref_k), 1e-6)
        assert rel.max() <= 2.0 ** -7, f"linear K row {L - 1} of sequence {b}: rel {rel.max():.2e}"
        assert torch.equal(vc[b, L - 1].cpu(), x["v_new"][b].cpu()), "linear V write"


def test_b64_decode_e4m3_linear_caches():
    """The bench's E4M3 decode step: the B=64 linear caches of the decode workload (same seed and
    draw) converted to E4M3 with zg_kv_to_fp8 (scale 1), then one ungated step through
    zg_attn_decode_fp8; every sequence against oracle.decode_fp8_cache over the same E4M3 values."""
    Bd, lo, hi = 64, 8192, 65536
    print(f"[case] E4M3 decode B={Bd} L~U[{lo},{hi}]", flush=True)
    x = si.decode_step(si.generator(1002, device=DEV), B=Bd, len_lo=lo, len_hi=hi, device=DEV)
    seq_h = x["seqlens"].cpu().numpy()
    kc8, vc8 = zg.zg_kv_to_fp8(x["lin_k"]), zg.zg_kv_to_fp8(x["lin_v"])
    del x["lin_k"], x["lin_v"], x["ring_k"], x["ring_v"]
    kc0 = {b: _host(kc8[b, :int(seq_h[b]) - 1]) for b in range(Bd)}  # rows before the new token
    vc0 = {b: _host(vc8[b, :int(seq_h[b]) - 1]) for b in range(Bd)}
    cfg = zg.AttnConfig(window=0, gated=False, rope_base=1e7)
    out = zg.zg_attn_decode_fp8(cfg, x["q_new"], x["k_new"], x["v_new"], None, kc8, vc8,
                                x["seqlens"], max_seqlen=hi)
    torch.cuda.synchronize()
    for b in range(Bd):
        L = int(seq_h[b])
        pad = np.zeros((1,) + kc0[b].shape[1:])
        r, _, rv = oracle.decode_fp8_cache(
            _host(x["q_new"][b:b + 1]), _host(x["k_new"][b:b + 1]), _host(x["v_new"][b:b + 1]),
            None, np.concatenate([kc0[b], pad])[None], np.concatenate([vc0[b], pad])[None],
            seq_h[b:b + 1], k_scale=1.0, v_scale=1.0, window=0, gated=False, rope_base=1e7)
        assert_parity(out[b:b + 1], r, f"E4M3 decode linear sequence {b} (L={L})")
        assert np.array_equal(_host(vc8[b, L - 1]), rv[0, L - 1]), f"E4M3 V row of sequence {b}"


@pytest.mark.parametrize("W", [128, 0])
def test_t262144_sampled_rows(W):
    T, base = 262144, 1e7
    print(f"[case] B=1 T={T} W={W} base={base}", flush=True)
    x = _layer(1, T, 1003, base)
    cfg = zg.AttnConfig(window=W, gated=W > 0, rope_base=base)
    out = zg.zg_attn_prefill(cfg, x["q"], x["k"], x["v"], x["gate"] if W else None)
    torch.cuda.synchronize()
    if W:
        rows = _rows(T, 256, 21)
        q, k, v, g = (_host(x[n]) for n in ("q", "k", "v", "gate"))
        ref = np.concatenate([oracle.prefill_rows(q, k, v, g, [r], window=W, gated=True,
                                                  rope_base=base) for r in rows], axis=1)
    else:
        rows = [0, 1, 127, 128, 129, 4095, 65536, 131071, 262143] + \
            np.random.default_rng(22).integers(0, T, 31).tolist()
        rows = sorted(set(rows))
        q, k, v = (_host(x[n]) for n in ("q", "k", "v"))
        ref = oracle.prefill_rows(q, k, v, None, rows, window=0, gated=False, rope_base=base)
    assert_parity(_host(out[:, rows]), ref, f"B=1 T=262144 W={W}, {len(rows)} rows")


@pytest.mark.parametrize("W", [128, 0])
def test_chunked_b4_ctx16384_sampled_rows(W):
    """zg_attn_prefill_cached with the inputs, caches and call of bench.py's chunked workload (same
    seed and draw order). The oracle row for new token t (position P = 16384 + t) is one decode
    step over the cache as it stands before P: the original cached rows for positions below 16384
    and, for 16384 .. P-1, the oracle's own k_hat and v of the new tokens."""
    Bc, ctx, Tc, base = 4, 16384, 2048, 1e6
    print(f"[case] chunked full size W={W}", flush=True)
    gen = si.generator(1005, device=DEV)
    x = si.prefill_layer(gen, Bc, Tc, 32, 8, 128, gated=True, device=DEV)
    for win in (0, 128):  # bench.py's draw order
        rows = win if win else ctx + Tc
        kc = si.randn_bf16(gen, (Bc, rows, 8, 128), device=DEV)
        vc = si.randn_bf16(gen, (Bc, rows, 8, 128), device=DEV)
        if win == W:
            break
    kc0, vc0 = kc.clone(), vc.clone()
    cfg = zg.AttnConfig(window=W, gated=W > 0, rope_base=base)
    need = zg.zg_attn_prefill_cached_workspace_bytes(cfg, Bc, Tc)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=DEV)
    out = zg.zg_attn_prefill_cached(cfg, x["q"], x["k"], x["v"], x["gate"] if W else None, kc, vc,
                                    pos0=ctx, workspace=ws)
    torch.cuda.synchronize()
    picks = [0, 1, 62, 63, 64, 126, 127, 128, 1023, 1024, 2046, 2047]
    picks += np.random.default_rng(31).integers(0, Tc, 3).tolist()
    picks = sorted(set(picks))
    got, ref = [], []
    for b in (0, Bc - 1):
        q, k, v, g = (_host(x[n][b]) for n in ("q", "k", "v", "gate"))
        k_cache, v_cache = _host(kc0[b]), _host(vc0[b])
        khat_new = oracle.qk_prologue(k, ctx + np.arange(Tc), None, rot_dim=42, rope_base=base,
                                      eps=1e-6)
        for t in picks:
            P = ctx + t
            kcb, vcb = k_cache.copy(), v_cache.copy()
            for p in range(max(ctx, P - W + 1) if W else ctx, P):
                slot = p % W if W else p
                kcb[slot], vcb[slot] = khat_new[p - ctx], v[p - ctx]
            o, _, _ = oracle.decode(q[t][None], k[t][None], v[t][None], g[t][None], kcb[None],
                                    vcb[None], np.array([P + 1]), window=W, gated=W > 0,
                                    rope_base=base)
            ref.append(o[0])
            got.append(_host(out[b, t]))
    assert_parity(np.stack(got), np.stack(ref),
                  f"chunked B=4 ctx=16384 +2048 W={W}, {len(picks)} rows x 2 sequences")


def test_stack_t65536_teacher_forced_layers():
    """The 32-layer stack's inputs as the benchmark draws them (seed 1004: x0, then each layer's
    weights in order) at T=65536, hidden 4096. All 32 layers run on the GPU in order; at layers 1
    and 32 (gated local) and 6 and 30 (global) the layer's sampled output rows are compared, as the
    layer's increment over its input, with oracle.stack_layer_rows applied to that same GPU input
    (teacher forcing). Global rows are sampled over the whole length (the oracle projects every key
    row below the last sampled one, about 1.1e12 fp64 FLOP per global layer), so the heaviest
    causal query tiles are among the compared rows."""
    Ts, hidden = 65536, 4096
    print(f"[case] stack layers 1, 6, 30 and 32, T={Ts}", flush=True)
    gen = si.generator(1004, device=DEV)
    x = si.stack_input(gen, 1, Ts, hidden, device=DEV)
    weights = [si.stack_layer_weights(gen, hidden, 32, 8, 128, is_global=(l % 6 == 0), device=DEV)
               for l in range(1, 33)]
    cfgs = {False: zg.AttnConfig(window=128, gated=True, rope_base=1e7),
            True: zg.AttnConfig(window=0, gated=False, rope_base=1e7)}
    ws = torch.empty(max(zg.zg_attn_layer_workspace_bytes(c, 1, Ts) for c in cfgs.values()),
                     dtype=torch.uint8, device=DEV)

    def run(l):
        g, w = l % 6 == 0, weights[l - 1]
        parts = [w["wq"], w["wk"], w["wv"]] + ([] if g else [w["wg"]])
        zg.zg_attn_layer(cfgs[g], x, torch.cat(parts, 0).contiguous(), w["wo"], workspace=ws)

    rng = np.random.default_rng(41)
    for l in range(1, 33):
        if l not in (1, 6, 30, 32):
            run(l)
            continue
        g = l % 6 == 0
        x_in = f64(x[0])
        run(l)
        torch.cuda.synchronize()
        edges = {0, 1, 2, 63, 64, 127, 128, 129, 1023, 1024, 2047, 4095, 32767, 32768, Ts - 65,
                 Ts - 64, Ts - 2, Ts - 1}
        rows = sorted(edges | set(rng.integers(0, Ts, 14 if g else 40).tolist()))
        w_h = {k: f64(v) for k, v in weights[l - 1].items()}
        ref = oracle.stack_layer_rows(x_in, w_h, rows, is_global=g, rope_base=1e7)
        got = f64(x[0, rows])
        assert_parity(got - x_in[rows], ref - x_in[rows],
                      f"stack layer {l} at T={Ts}, {len(rows)} rows")
        del x_in, w_h, ref
