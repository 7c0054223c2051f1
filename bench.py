#!/usr/bin/env python3
"""Benchmark of the ZGCM-1 hybrid attention core on one MI355X.

Step = one pass of the prefill hot path over the B=4 x T=16384 batch (the pages' pre-training
length): five gated sliding-window layers (W=128) and one full-causal global layer, the repeating
5:1 block of the model (ZGCM-1 zh-TW translation page, section 2.1). Every layer runs the whole
fused path: QK-RMSNorm + partial RoPE (rot 42, base 1e6), banded/causal GQA attention with online
softmax on bf16 MFMA, sigmoid gate. value = B*T / (time of one block) in tokens/s.

Also measured in the same run (reported beside the headline):
  * the B=64 decode step over a 128-slot ring (local layer) and a linear cache with context lengths
    uniform on [8192, 65536] (global layer), cold caches, as GB/s of KV read against HBM peak; the
    linear step again over E4M3 caches;
  * one gated local and one global layer at B=1, T=262144 (base 1e7), against the HBM and MFMA
    rooflines;
  * the 32-layer attention stack with projections at B=1, T=65536 (27 gated local + 5 global
    layers, hidden 4096, N(0, 0.02) weights), as tokens/s and useful TFLOP/s with a per-component
    breakdown;
  * chunked prefill through the decode caches: B=4 sequences continue with 2048 new tokens after
    16384 cached positions, on a global layer (linear caches) and a gated local layer (rings);
  * a context sweep at 262,144 tokens per step (T = 4K .. 256K, B = 256K / T): one local and one
    global layer timed per T, and the 32-layer attention time of the all-global, 1:1, 3:1 and
    ZGCM-1's 5:1 schedules (global at every 1st, 2nd, 4th, 6th layer);
  * the B=1, T=1024 gated local layer (cold MALL);
  * the oracle (fp64 NumPy on the host cores) on a bounded sample of the same workload, and on
    samples of the other workloads (per-config rates, scaled-up figures labelled extrapolated).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode] [--no-long]
                       [--no-stack] [--no-chunked] [--no-sweep] [--no-block]
Prints ONE JSON line on stdout.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15    # FLOP/s, MI355X dense bf16
B, T, HQ, HKV, D, W = 4, 16384, 32, 8, 128, 128
ROPE_BASE = 1e6
SEED = 1001


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def n_pairs(T, W):
    """(query, key) pairs per head and sequence of a window-W (0: causal) layer."""
    if 0 < W < T:
        return W * (W + 1) // 2 + (T - W) * W
    return T * (T + 1) // 2


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-reps", type=int, default=20)
    ap.add_argument("--no-long", action="store_true", help="skip the B=1, T=262144 layers")
    ap.add_argument("--no-stack", action="store_true", help="skip the 32-layer stack")
    ap.add_argument("--no-chunked", action="store_true", help="skip the chunked prefill")
    ap.add_argument("--no-sweep", action="store_true", help="skip the context sweep")
    ap.add_argument("--no-backward", action="store_true", help="skip the training (backward) layers")
    ap.add_argument("--no-shard", action="store_true", help="skip the one-GPU-share layers")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the timed 5:1 block (profiling the other workloads alone; value null)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the attention core shards by (batch x KV head) with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import global_causal_attention_amd as zg
    import synth_inputs as si

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    log(f"[bench] device {torch.cuda.get_device_name(0)}")

    result = {
        "metric": "gated-SWA/global attn prefill tokens/s + %MFMA peak; decode HBM GB/s %peak",
        "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "hybrid 5:1 prefill block (5 gated-SWA W=128 + 1 global causal "
                               "layer), B=4 T=16384 Hq=32 Hkv=8 D=128, rot 42 base 1e6",
                   "global_batch": B, "seq_len": T, "parallelism": "none (1 GPU)"}}
    if not args.no_block:
        result.update(bench_block(torch, zg, si, dev, stream, args))

    if not args.no_decode:
        result["decode"] = bench_decode(torch, zg, si, dev, stream, args.decode_reps)
        result["t1024_local"] = bench_t1024(torch, zg, si, dev, stream)
    if not args.no_long:
        result["long_context"] = bench_long(torch, zg, si, dev, stream)
    if not args.no_stack:
        result["stack"] = bench_stack(torch, zg, si, dev, stream)
    if not args.no_chunked:
        result["chunked_prefill"] = bench_chunked(torch, zg, si, dev, stream)
    if not args.no_sweep:
        result["context_sweep"] = bench_sweep(torch, zg, si, dev, stream)
    if not args.no_backward:
        result["training"] = bench_backward(torch, zg, si, dev, stream)
    if not args.no_shard:
        full = None
        if "swa_ms" in result.get("layers", {}):
            full = {"swa": result["layers"]["swa_ms"], "global": result["layers"]["global_ms"]}
        result["shard_share"] = bench_shard(torch, zg, si, dev, stream, full)

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(torch, si)
        result["cpu_baseline_configs"] = cpu_baseline_configs(torch, si)

    print(json.dumps(result), flush=True)


def bench_block(torch, zg, si, dev, stream, args):
    """The timed 5:1 block at B=4, T=16384 (the headline value and roofline)."""
    log(f"[bench] building inputs B={B} T={T}")
    gen = si.generator(SEED, device="cuda")
    swa = si.prefill_layer(gen, B, T, HQ, HKV, D, gated=True, device="cuda")
    glo = si.prefill_layer(gen, B, T, HQ, HKV, D, gated=False, device="cuda")
    cfg_swa = zg.AttnConfig(window=W, gated=True, rope_base=ROPE_BASE)
    cfg_glo = zg.AttnConfig(window=0, gated=False, rope_base=ROPE_BASE)
    out_swa = torch.empty_like(swa["q"])
    out_glo = torch.empty_like(glo["q"])
    ws = torch.empty(max(zg.zg_attn_prefill_workspace_bytes(c, B, T) for c in (cfg_swa, cfg_glo)),
                     dtype=torch.uint8, device=dev)

    def run_swa():
        zg.zg_attn_prefill(cfg_swa, swa["q"], swa["k"], swa["v"], swa["gate"], out=out_swa,
                           workspace=ws)

    def run_glo():
        zg.zg_attn_prefill(cfg_glo, glo["q"], glo["k"], glo["v"], out=out_glo, workspace=ws)

    # calibration copy for HBM counters (a plain 1 GiB device copy, outside the timed region)
    calib_src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    del calib_src, calib_dst

    for _ in range(args.warmup):
        for _ in range(5):
            run_swa()
        run_glo()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(K)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(K):
        ev[s][0].record(stream)
        for i in range(5):
            run_swa()
            ev[s][i + 1].record(stream)
        run_glo()
        ev[s][6].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / K
    # the global layer again, five launches back to back (reported beside the block timing)
    e_b2b = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    e_b2b[0].record(stream)
    for i in range(5):
        run_glo()
        e_b2b[i + 1].record(stream)
    torch.cuda.synchronize()
    glo_b2b = sorted(e_b2b[i].elapsed_time(e_b2b[i + 1]) for i in range(5))[2]
    swa_ms = sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(K) for i in range(5)) / (5 * K)
    glo_ms = sum(ev[s][5].elapsed_time(ev[s][6]) for s in range(K)) / K
    tokens = B * T
    value = tokens / (ms_step * 1e-3)

    flop_pair = 4 * D
    glo_flop = B * HQ * n_pairs(T, 0) * flop_pair
    swa_flop = B * HQ * n_pairs(T, W) * flop_pair
    swa_bytes = B * T * (HQ * D * 2 * 3 + HKV * D * 2 * 2)   # q, gate, out + k, v (bf16)
    glo_achieved = glo_flop / (glo_ms * 1e-3)
    # HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE record (null if the kernels
    # changed since it was taken)
    from global_causal_attention_amd.counters import lookup_traffic
    # threads: 64-query tiles x (b, kv head) workgroups of 512, or one workgroup per CU walking
    # them when the layer has at least two tiles per CU (the library's persistent launch)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    tiles = ((T + 63) // 64) * B * HKV
    grid_prefill = (cus if (tiles >= 2 * cus and cus % 8 == 0) else tiles) * 512
    grid_kprep = min((B * T * HKV + 31) // 32, 2048) * 256  # threads: 32 rows per block pass
    parts = [lookup_traffic("prefill_kernel<4, false>", grid_prefill),
             lookup_traffic("kprep_kernel", grid_kprep)]
    glo_traffic = None if None in parts else sum(parts)
    result = {
        "value": round(value, 1),
        "ms_per_step": round(ms_step, 4),
        "roofline": {"bound": "mfma", "achieved": round(glo_achieved / 1e12, 2),
                     "peak": MFMA_BF16_PEAK / 1e12, "unit": "TFLOP/s",
                     "frac": round(glo_achieved / MFMA_BF16_PEAK, 4),
                     "traffic": glo_traffic,
                     "kernel": "global causal prefill launch (kprep_kernel + "
                               "prefill_kernel<4, false>)",
                     "flop_per_launch": glo_flop},
        "layers": {
            "swa_ms": round(swa_ms, 4), "global_ms": round(glo_ms, 4),
            "weighted_5to1_ms": round(5 * swa_ms + glo_ms, 4),
            "swa_hbm_GBps": round(swa_bytes / (swa_ms * 1e-3) / 1e9, 1),
            "swa_hbm_frac": round(swa_bytes / (swa_ms * 1e-3) / HBM_PEAK, 4),
            "swa_min_bytes": swa_bytes,
            "swa_mfma_TFLOPs_useful": round(swa_flop / (swa_ms * 1e-3) / 1e12, 2),
            "global_TFLOPs": round(glo_achieved / 1e12, 2),
            "global_back_to_back_ms": round(glo_b2b, 4),
            "global_back_to_back_mfma_frac": round(glo_flop / (glo_b2b * 1e-3) / MFMA_BF16_PEAK, 4),
            "global_tokens_per_s": round(tokens / (glo_ms * 1e-3), 1),
            "swa_tokens_per_s": round(tokens / (swa_ms * 1e-3), 1),
        },
    }
    log(f"[bench] step {ms_step:.3f} ms; swa {swa_ms:.3f} ms; global {glo_ms:.3f} ms")
    del swa, glo, out_swa, out_glo, ws
    return result


def bench_t1024(torch, zg, si, dev, stream, reps=20):
    """The small check workload timed: one gated local layer, B=1, T=1024 (W=128, base 1e4, seed
    1000). Its 29.4 MB of inputs and outputs fit the MALL, so each rep starts after a 1 GiB fill
    that evicts them (cold); median of `reps`."""
    x = si.prefill_layer(si.generator(1000, device="cuda"), 1, 1024, HQ, HKV, D, gated=True,
                         device="cuda")
    cfg = zg.AttnConfig(window=W, gated=True, rope_base=1e4)
    out = torch.empty_like(x["q"])
    ws = torch.empty(zg.zg_attn_prefill_workspace_bytes(cfg, 1, 1024), dtype=torch.uint8, device=dev)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    fn = lambda: zg.zg_attn_prefill(cfg, x["q"], x["k"], x["v"], x["gate"], out=out, workspace=ws)
    for _ in range(3):
        fn()
    ts = []
    for _ in range(reps):
        flush.fill_(1)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ts.sort()
    ms = ts[len(ts) // 2]
    nbytes = 1024 * (HQ * D * 2 * 3 + HKV * D * 2 * 2)
    log(f"[bench] T=1024 local layer: {ms * 1e3:.1f} us")
    del x, out, ws, flush
    return {"workload": "B=1, T=1024, Hq=32 Hkv=8 D=128, gated W=128, rot 42, base 1e4, cold MALL",
            "ms_median": round(ms, 4), "tokens_per_s": round(1024 / (ms * 1e-3), 1),
            "min_bytes": nbytes, "hbm_frac": round(nbytes / (ms * 1e-3) / HBM_PEAK, 4)}


def bench_decode(torch, zg, si, dev, stream, reps):
    """B=64 decode step: ring (local) and linear (global) layers; MALL/L2 flushed before each rep."""
    Bd, lo, hi = 64, 8192, 65536
    gen = si.generator(1002, device="cuda")
    log("[bench] building decode caches (2 x 8 GiB linear, 2 x 16 MiB ring)")
    x = si.decode_step(gen, B=Bd, len_lo=lo, len_hi=hi, device="cuda")
    seqlens = x["seqlens"]
    sum_len = int(seqlens.sum().item())
    cfg_r = zg.AttnConfig(window=W, gated=True, rope_base=1e7)
    cfg_l = zg.AttnConfig(window=0, gated=False, rope_base=1e7)
    ws_r = torch.empty(zg.zg_attn_decode_workspace_bytes(cfg_r, Bd, hi), dtype=torch.uint8, device=dev)
    ws_l = torch.empty(zg.zg_attn_decode_workspace_bytes(cfg_l, Bd, hi), dtype=torch.uint8, device=dev)
    out = torch.empty_like(x["q_new"])
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def ring():
        zg.zg_attn_decode(cfg_r, x["q_new"], x["k_new"], x["v_new"], x["gate"], x["ring_k"],
                          x["ring_v"], seqlens, max_seqlen=hi, out=out, workspace=ws_r)

    def lin():
        zg.zg_attn_decode(cfg_l, x["q_new"], x["k_new"], x["v_new"], None, x["lin_k"],
                          x["lin_v"], seqlens, max_seqlen=hi, out=out, workspace=ws_l)

    res = {}
    for name, fn, kv_bytes in (("ring", ring, Bd * W * HKV * D * 2 * 2),
                               ("linear", lin, sum_len * HKV * D * 2 * 2)):
        for _ in range(3):
            fn()
        times = []
        for _ in range(reps):
            flush.fill_(1)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        times.sort()
        med = times[len(times) // 2]
        bw = kv_bytes / (med * 1e-3)
        res[name] = {"ms_median": round(med, 4), "kv_bytes": kv_bytes, "GBps": round(bw / 1e9, 1),
                     "hbm_frac": round(bw / HBM_PEAK, 4), "tokens_per_s": round(Bd / (med * 1e-3), 1)}
        log(f"[bench] decode {name}: {med:.4f} ms, {bw / 1e9:.1f} GB/s")
    # The local layers of one decode step (27 of a 32-layer 5:1 stack) run back to back, each over
    # its own ring cache (27 x 32 MiB, so every layer starts cold): per-layer time of that sequence.
    # The isolated call above also holds the event and dispatch overhead around one short kernel.
    n_local = 27
    rings = [(si.randn_bf16(gen, x["ring_k"].shape, device=dev),
              si.randn_bf16(gen, x["ring_v"].shape, device=dev)) for _ in range(n_local)]
    outs = [torch.empty_like(x["q_new"]) for _ in range(n_local)]

    def ring_layers():
        for (rk, rv), o in zip(rings, outs):
            zg.zg_attn_decode(cfg_r, x["q_new"], x["k_new"], x["v_new"], x["gate"], rk, rv, seqlens,
                              max_seqlen=hi, out=o, workspace=ws_r)

    ring_layers()
    times = []
    for _ in range(reps):
        for _ in range(6):
            flush.fill_(1)  # ~1.2 ms of device work while the host enqueues the 27 calls
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        ring_layers()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / n_local)
    times.sort()
    med = times[len(times) // 2]
    kvb = res["ring"]["kv_bytes"]
    res["ring"]["back_to_back"] = {
        "layers": n_local, "ms_per_layer_median": round(med, 4),
        "GBps": round(kvb / (med * 1e-3) / 1e9, 1), "hbm_frac": round(kvb / (med * 1e-3) / HBM_PEAK, 4)}
    log(f"[bench] decode ring, {n_local} layers back to back: {med * 1e3:.2f} us per layer")
    del rings, outs
    # streaming-read reference: the probe reads the 8 GiB linear K cache (cold MALL) with the same
    # non-temporal 16-byte loads the decode kernels use
    sink = torch.empty(4 * 2048, dtype=torch.int32, device=dev)
    pbytes = x["lin_k"].numel() * x["lin_k"].element_size()
    zg.zg_hbm_read_probe(x["lin_k"], sink)
    ptimes = []
    for _ in range(5):
        flush.fill_(1)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        zg.zg_hbm_read_probe(x["lin_k"], sink)
        e1.record(stream)
        torch.cuda.synchronize()
        ptimes.append(e0.elapsed_time(e1))
    ptimes.sort()
    pbw = pbytes / (ptimes[2] * 1e-3)
    res["read_probe"] = {"bytes": pbytes, "ms_median": round(ptimes[2], 4),
                         "GBps": round(pbw / 1e9, 1), "frac_of_spec": round(pbw / HBM_PEAK, 4)}
    for name in ("ring", "linear"):
        res[name]["frac_of_read_probe"] = round(res[name]["GBps"] * 1e9 / pbw, 4)
    log(f"[bench] streaming read probe: {pbw / 1e9:.1f} GB/s")
    # the same step over E4M3 caches (converted once from the bf16 ones, outside the timing)
    lin_k8 = zg.zg_kv_to_fp8(x["lin_k"])
    lin_v8 = zg.zg_kv_to_fp8(x["lin_v"])

    def lin8():
        zg.zg_attn_decode_fp8(cfg_l, x["q_new"], x["k_new"], x["v_new"], None, lin_k8, lin_v8,
                              seqlens, max_seqlen=hi, out=out, workspace=ws_l)

    for _ in range(3):
        lin8()
    times = []
    for _ in range(reps):
        flush.fill_(1)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        lin8()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    times.sort()
    med = times[len(times) // 2]
    kv8 = sum_len * HKV * D * 2
    res["linear_e4m3"] = {"ms_median": round(med, 4), "kv_bytes": kv8,
                          "GBps": round(kv8 / (med * 1e-3) / 1e9, 1),
                          "hbm_frac": round(kv8 / (med * 1e-3) / HBM_PEAK, 4),
                          "tokens_per_s": round(Bd / (med * 1e-3), 1),
                          "speedup_vs_bf16": round(res["linear"]["ms_median"] / med, 3),
                          "frac_of_read_probe": round(kv8 / (med * 1e-3) / pbw, 4)}
    log(f"[bench] decode linear E4M3: {med:.4f} ms, {kv8 / (med * 1e-3) / 1e9:.1f} GB/s")
    del lin_k8, lin_v8
    res["workload"] = "B=64, Hq=32 Hkv=8 D=128, ring W=128 gated; linear L~U[8192,65536] ungated; base 1e7; cold MALL"
    from global_causal_attention_amd.counters import lookup_traffic
    parts = [lookup_traffic("decode_prep_kernel", ((Bd * (HQ + HKV) + 15) // 16) * 256),
             lookup_traffic("decode_mfma_kernel<false>", Bd * HKV * 16 * 1024),
             lookup_traffic("decode_combine_kernel", 262144)]
    res["roofline"] = {"bound": "hbm", "achieved": res["linear"]["GBps"], "peak": HBM_PEAK / 1e9,
                       "unit": "GB/s", "frac": res["linear"]["hbm_frac"],
                       "traffic": None if None in parts else sum(parts),
                       "kernel": "global decode launch (decode_prep_kernel + "
                                 "decode_mfma_kernel<false> + decode_combine_kernel)"}
    del x, flush
    return res


_BUSY = {}


def _time(torch, stream, fn, reps, warm=1):
    """Median of `reps` timed calls (HIP events on the launch stream) after `warm` untimed ones.
    Before each call the stream is kept busy by a 1 GiB device fill (about 0.2 ms), so the host
    has enqueued the call's launches before the start event executes: the interval holds the
    call's GPU work only, not the host's launch latency (which would dominate calls of ~0.1 ms).
    The fill also leaves the caches cold, as in the decode timings."""
    busy = _BUSY.get(stream.device)
    if busy is None:
        busy = _BUSY[stream.device] = torch.empty(1 << 30, dtype=torch.uint8, device=stream.device)
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        busy.fill_(1)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ts.sort()
    return ts[len(ts) // 2]


def bench_long(torch, zg, si, dev, stream):
    """B=1, T=262144: one gated local layer (W=128) and one global layer, RoPE base 1e7."""
    Tl = 262144
    log(f"[bench] long context: building B=1 T={Tl} layer inputs")
    x = si.prefill_layer(si.generator(1003, device="cuda"), 1, Tl, HQ, HKV, D, gated=True,
                         device="cuda")
    out = torch.empty_like(x["q"])
    res = {"workload": f"B=1, T={Tl}, Hq=32 Hkv=8 D=128, rot 42, base 1e7"}
    for name, win in (("swa", W), ("global", 0)):
        cfg = zg.AttnConfig(window=win, gated=win > 0, rope_base=1e7)
        ws = torch.empty(zg.zg_attn_prefill_workspace_bytes(cfg, 1, Tl), dtype=torch.uint8, device=dev)
        fn = lambda: zg.zg_attn_prefill(cfg, x["q"], x["k"], x["v"], x["gate"] if win else None,
                                        out=out, workspace=ws)
        ms = _time(torch, stream, fn, 5)
        flop = HQ * n_pairs(Tl, win) * 4 * D
        r = {"ms_median": round(ms, 3), "tokens_per_s": round(Tl / (ms * 1e-3), 1),
             "TFLOPs_useful": round(flop / (ms * 1e-3) / 1e12, 2)}
        if win:
            nbytes = Tl * (HQ * D * 2 * 3 + HKV * D * 2 * 2)
            r.update({"min_bytes": nbytes, "hbm_frac": round(nbytes / (ms * 1e-3) / HBM_PEAK, 4)})
        else:
            r["mfma_frac"] = round(flop / (ms * 1e-3) / MFMA_BF16_PEAK, 4)
        res[name] = r
        log(f"[bench] T={Tl} {name}: {ms:.3f} ms")
        del ws
    del x, out
    return res


def bench_stack(torch, zg, si, dev, stream, n_layers=32, Ts=65536, hidden=4096):
    """The attention-only stack with projections: x <- x + o_proj(attn(RMSNorm(x))) for 32 layers,
    global at layers 6, 12, 18, 24, 30 (ungated, full causal), gated W=128 elsewhere; base 1e7.
    One untimed pass, then five timed passes (the fastest is reported; the median beside it);
    per-layer events give the breakdown."""
    log(f"[bench] stack: {n_layers} layers, T={Ts}, hidden {hidden}")
    gen = si.generator(1004, device="cuda")
    x = si.stack_input(gen, 1, Ts, hidden, device="cuda")
    layers = []
    for l in range(1, n_layers + 1):
        g = l % 6 == 0
        w = si.stack_layer_weights(gen, hidden, HQ, HKV, D, is_global=g, device="cuda")
        parts = [w["wq"], w["wk"], w["wv"]] + ([] if g else [w["wg"]])
        layers.append((g, torch.cat(parts, 0).contiguous(), w["wo"]))
        del w, parts
    cfgs = {False: zg.AttnConfig(window=W, gated=True, rope_base=1e7),
            True: zg.AttnConfig(window=0, gated=False, rope_base=1e7)}
    ws = torch.empty(max(zg.zg_attn_layer_workspace_bytes(c, 1, Ts) for c in cfgs.values()),
                     dtype=torch.uint8, device=dev)

    def timed(run_layer):
        """One untimed pass, then five timed ones: (fastest total, its per-layer ms, median)."""
        def one_pass(evs=None):
            for i, lay in enumerate(layers):
                run_layer(lay)
                if evs is not None:
                    evs[i + 1].record(stream)

        one_pass()
        torch.cuda.synchronize()
        runs = []
        for _ in range(5):
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_layers + 1)]
            evs[0].record(stream)
            one_pass(evs)
            torch.cuda.synchronize()
            per = [evs[i].elapsed_time(evs[i + 1]) for i in range(n_layers)]
            runs.append((sum(per), per))
        runs.sort(key=lambda r: r[0])
        return runs[0][0], runs[0][1], runs[len(runs) // 2][0]

    total, per, median_ms = timed(lambda lay: zg.zg_attn_layer(cfgs[lay[0]], x, lay[1], lay[2],
                                                               workspace=ws))
    n_glob = sum(1 for g, _, _ in layers if g)
    t_glob = sum(p for p, (g, _, _) in zip(per, layers) if g)
    t_loc = total - t_glob
    # useful FLOP: projections (2 per weight per token) + attention (4*D per (head, key) pair)
    proj = sum(2 * Ts * (wqkvg.numel() + wo.numel()) for _, wqkvg, wo in layers)
    att = sum(HQ * n_pairs(Ts, 0 if g else W) * 4 * D for g, _, _ in layers)
    res = {"workload": f"B=1, T={Ts}, hidden {hidden}, {n_layers} layers ({n_glob} global), "
                       f"N(0, 0.02) bf16 weights, fp32 residual, base 1e7",
           "ms": round(total, 2), "ms_median_of_5": round(median_ms, 2),
           "tokens_per_s": round(Ts / (total * 1e-3), 1),
           "useful_flop": proj + att,
           "TFLOPs_useful": round((proj + att) / (total * 1e-3) / 1e12, 1),
           "mfma_frac": round((proj + att) / (total * 1e-3) / MFMA_BF16_PEAK, 4),
           "local_layer_ms": round(t_loc / (n_layers - n_glob), 3),
           "global_layer_ms": round(t_glob / n_glob, 3)}

    # the same layers with E4M3 projections: weights quantized per output row once (untimed);
    # inside each layer the hidden state and the attention output are quantized per row
    log("[bench] stack with E4M3 projections")
    layers8 = []
    for g, wqkvg, wo in layers:
        cq, sq = zg.zg_quant_rows_fp8(wqkvg)
        co, so = zg.zg_quant_rows_fp8(wo)
        layers8.append((g, cq, sq, co, so))
    del ws
    ws8 = torch.empty(max(zg.zg_attn_layer_fp8_workspace_bytes(c, 1, Ts) for c in cfgs.values()),
                      dtype=torch.uint8, device=dev)
    lay8 = {id(l): l8 for l, l8 in zip(layers, layers8)}
    total8, per8, median8 = timed(lambda lay: zg.zg_attn_layer_fp8(
        cfgs[lay[0]], x, *lay8[id(lay)][1:], workspace=ws8))
    t_glob8 = sum(p for p, (g, _, _) in zip(per8, layers) if g)
    res["e4m3_projections"] = {
        "ms": round(total8, 2), "ms_median_of_5": round(median8, 2),
        "tokens_per_s": round(Ts / (total8 * 1e-3), 1),
        "speedup_vs_bf16": round(total / total8, 3),
        "local_layer_ms": round((total8 - t_glob8) / (n_layers - n_glob), 3),
        "global_layer_ms": round(t_glob8 / n_glob, 3),
        "note": "projections on E4M3 operands (per-row scales, fp32 accumulation), attention bf16"}
    log(f"[bench] stack: bf16 {total:.1f} ms, E4M3 projections {total8:.1f} ms")
    del layers, layers8, ws8, x
    return res


def bench_chunked(torch, zg, si, dev, stream, Bc=4, ctx=16384, Tc=2048):
    """Chunked prefill through the caches: each of Bc sequences has ctx positions in its caches and
    continues with Tc new tokens (base 1e6). Cache contents are N(0,1) bf16 standing for
    normalised, rotated keys and values; every timed call rewrites the same cache rows."""
    log(f"[bench] chunked prefill: B={Bc}, {ctx} cached positions + {Tc} new")
    gen = si.generator(1005, device="cuda")
    x = si.prefill_layer(gen, Bc, Tc, HQ, HKV, D, gated=True, device="cuda")
    out = torch.empty_like(x["q"])
    res = {"workload": f"B={Bc}, {ctx} cached positions + {Tc} new tokens, Hq=32 Hkv=8 D=128, "
                       f"base 1e6; global layer on linear caches, gated W=128 layer on rings"}
    for name, win in (("global", 0), ("swa", W)):
        rows = win if win else ctx + Tc
        kc = si.randn_bf16(gen, (Bc, rows, HKV, D), device="cuda")
        vc = si.randn_bf16(gen, (Bc, rows, HKV, D), device="cuda")
        cfg = zg.AttnConfig(window=win, gated=win > 0, rope_base=ROPE_BASE)
        need = zg.zg_attn_prefill_cached_workspace_bytes(cfg, Bc, Tc)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        fn = lambda: zg.zg_attn_prefill_cached(cfg, x["q"], x["k"], x["v"],
                                               x["gate"] if win else None, kc, vc, pos0=ctx,
                                               out=out, workspace=ws)
        ms = _time(torch, stream, fn, 10)
        if win:
            pairs = Tc * win   # every new query sees a full window
            nbytes = Bc * Tc * (HQ * D * 2 * 3 + HKV * D * 2 * 2) + Bc * min(Tc, win) * HKV * D * 2 * 2
            r = {"ms_median": round(ms, 4), "hbm_frac": round(nbytes / (ms * 1e-3) / HBM_PEAK, 4),
                 "min_bytes": nbytes}
        else:
            pairs = Tc * ctx + Tc * (Tc + 1) // 2
            flop = Bc * HQ * pairs * 4 * D
            r = {"ms_median": round(ms, 4), "TFLOPs_useful": round(flop / (ms * 1e-3) / 1e12, 1),
                 "mfma_frac": round(flop / (ms * 1e-3) / MFMA_BF16_PEAK, 4)}
        r["tokens_per_s"] = round(Bc * Tc / (ms * 1e-3), 1)
        res[name] = r
        log(f"[bench] chunked {name}: {ms:.3f} ms")
        del kc, vc, ws
    del x, out
    return res


def bench_backward(torch, zg, si, dev, stream, Bb=B, Tb=T):
    """Training layers at the prefill shape: forward with the row log-sum-exp, then the backward
    pass (dq, dk, dv, dgate), for a gated local layer (W=128) and an ungated global layer (base
    1e6). FLOPs follow the usual convention: forward 4 D per (query, key) pair and head, backward
    2.5 times that (the score recomputation included). The local layer's minimum HBM traffic is
    its inputs and outputs once: q, gate, out, dout, dq, dgate ([B, T, Hq, D] bf16), k, v, dk, dv
    ([B, T, Hkv, D] bf16) and lse."""
    log(f"[bench] training layers: B={Bb} T={Tb}")
    gen = si.generator(1007, device="cuda")
    res = {"workload": f"B={Bb}, T={Tb}, Hq=32 Hkv=8 D=128, rot 42, base 1e6: forward with "
                       f"log-sum-exp + backward (dq, dk, dv, dgate)"}
    total = 0.0
    for name, win in (("swa", W), ("global", 0)):
        x = si.prefill_layer(gen, Bb, Tb, HQ, HKV, D, gated=win > 0, device="cuda")
        dy = si.randn_bf16(gen, (Bb, Tb, HQ, D), device="cuda")
        cfg = zg.AttnConfig(window=win, gated=win > 0, rope_base=ROPE_BASE)
        g = x["gate"] if win else None
        out, lse = zg.zg_attn_forward_train(cfg, x["q"], x["k"], x["v"], g)
        fws = torch.empty(zg.zg_attn_forward_train_workspace_bytes(cfg, Bb, Tb), dtype=torch.uint8,
                          device=dev)
        bws = torch.empty(zg.zg_attn_backward_workspace_bytes(cfg, Bb, Tb), dtype=torch.uint8, device=dev)
        f_ms = _time(torch, stream, lambda: zg.zg_attn_forward_train(
            cfg, x["q"], x["k"], x["v"], g, out=out, lse=lse, workspace=fws), 5)
        b_ms = _time(torch, stream, lambda: zg.zg_attn_backward(
            cfg, x["q"], x["k"], x["v"], g, out, dy, lse, workspace=bws), 5)
        flop = Bb * HQ * n_pairs(Tb, win) * 4 * D
        r = {"fwd_ms": round(f_ms, 3), "bwd_ms": round(b_ms, 3),
             "bwd_TFLOPs": round(2.5 * flop / (b_ms * 1e-3) / 1e12, 1),
             "bwd_mfma_frac": round(2.5 * flop / (b_ms * 1e-3) / MFMA_BF16_PEAK, 4)}
        if win:
            nbytes = Bb * Tb * (HQ * D * 2 * 6 + HKV * D * 2 * 4 + HQ * 4)
            r.update({"bwd_min_bytes": nbytes, "bwd_hbm_frac": round(nbytes / (b_ms * 1e-3) / HBM_PEAK, 4)})
        res[name] = r
        total += (5 if win else 1) * (f_ms + b_ms)
        log(f"[bench] training {name}: fwd {f_ms:.3f} ms, bwd {b_ms:.3f} ms")
        del x, dy, out, lse, fws, bws
    res["block_5to1_ms"] = round(total, 3)
    res["block_5to1_tokens_per_s"] = round(Bb * Tb / (total * 1e-3), 1)
    return res


def bench_shard(torch, zg, si, dev, stream, full_ms=None, Bs=B, Ts=T):
    """One GPU's share of a layer when the attention core is split over the 8 KV-head groups
    (4 query heads, 1 KV head, no exchange): B=4, T=16384, one gated local and one global layer
    (base 1e6). `vs_eighth_of_full` compares with 1/8 of the full layer's time from the block
    when that section ran."""
    log(f"[bench] one-GPU share: B={Bs} T={Ts} Hq=4 Hkv=1")
    x = si.prefill_layer(si.generator(1008, device="cuda"), Bs, Ts, 4, 1, D, gated=True,
                         device="cuda")
    out = torch.empty_like(x["q"])
    res = {"workload": f"B={Bs}, T={Ts}, Hq=4 Hkv=1 D=128 (one KV-head group of 8), base 1e6"}
    for name, win in (("swa", W), ("global", 0)):
        cfg = zg.AttnConfig(n_q_heads=4, n_kv_heads=1, window=win, gated=win > 0,
                            rope_base=ROPE_BASE)
        ws = torch.empty(zg.zg_attn_prefill_workspace_bytes(cfg, Bs, Ts), dtype=torch.uint8, device=dev)
        fn = lambda: zg.zg_attn_prefill(cfg, x["q"], x["k"], x["v"], x["gate"] if win else None,
                                        out=out, workspace=ws)
        ms = _time(torch, stream, fn, 10)
        r = {"ms_median": round(ms, 4), "tokens_per_s": round(Bs * Ts / (ms * 1e-3), 1)}
        flop = Bs * 4 * n_pairs(Ts, win) * 4 * D
        if win:
            nbytes = Bs * Ts * (4 * D * 2 * 3 + D * 2 * 2)
            r["hbm_frac"] = round(nbytes / (ms * 1e-3) / HBM_PEAK, 4)
        else:
            r["mfma_frac"] = round(flop / (ms * 1e-3) / MFMA_BF16_PEAK, 4)
        if full_ms and name in full_ms:
            r["vs_eighth_of_full"] = round(full_ms[name] / 8 / ms, 4)
        res[name] = r
        log(f"[bench] share {name}: {ms:.4f} ms")
        del ws
    del x, out
    return res


def bench_sweep(torch, zg, si, dev, stream, tokens=262144, n_layers=32):
    """Attention-only context sweep at a fixed number of tokens per step: per T, one gated local
    layer (W=128) and one global layer are timed (base 1e7); a schedule's 32-layer attention time
    is n_local * t_local + n_global * t_global, with layer l global iff l % every == 0."""
    res = {"workload": f"{tokens} tokens per step, B = {tokens} / T, Hq=32 Hkv=8 D=128, base 1e7",
           "points": []}
    schedules = {"all_global": 1, "1:1": 2, "3:1": 4, "5:1": 6}
    for T_ in (4096, 8192, 16384, 32768, 65536, 131072, 262144):
        Bs = tokens // T_
        x = si.prefill_layer(si.generator(1006, device="cuda"), Bs, T_, HQ, HKV, D, gated=True,
                             device="cuda")
        out = torch.empty_like(x["q"])
        t = {}
        for name, win in (("local", W), ("global", 0)):
            cfg = zg.AttnConfig(window=win, gated=win > 0, rope_base=1e7)
            ws = torch.empty(zg.zg_attn_prefill_workspace_bytes(cfg, Bs, T_), dtype=torch.uint8,
                             device=dev)
            fn = lambda: zg.zg_attn_prefill(cfg, x["q"], x["k"], x["v"], x["gate"] if win else None,
                                            out=out, workspace=ws)
            t[name] = _time(torch, stream, fn, 3 if win else 2)
            del ws
        del x, out
        point = {"T": T_, "B": Bs, "local_ms": round(t["local"], 3), "global_ms": round(t["global"], 3)}
        for sname, every in schedules.items():
            n_g = n_layers // every  # layers 1..n_layers that are multiples of `every`
            ms = (n_layers - n_g) * t["local"] + n_g * t["global"]
            point[sname] = {"n_global": n_g, "ms": round(ms, 2), "tokens_per_s": round(tokens / (ms * 1e-3), 1)}
        point["5:1_vs_all_global"] = round(point["all_global"]["ms"] / point["5:1"]["ms"], 3)
        res["points"].append(point)
        log(f"[bench] sweep T={T_}: local {t['local']:.3f} ms, global {t['global']:.3f} ms")
    return res


def _oracle_threads():
    """BLAS threads for the oracle: every core this process may run on."""
    n = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(n)
    except Exception:
        pass
    return n


def cpu_baseline_configs(torch, si, budget_s=8.0):
    """The oracle (fp64 NumPy on the host cores) on the other workloads, each on a bounded sample
    with the shapes of the GPU workload (inputs drawn on the host; the oracle's time does not depend
    on the values). Rates are in the unit of the GPU figure they sit beside; every figure that is
    scaled up from a sample says so."""
    import numpy as np
    import oracle
    cores = _oracle_threads()
    f = lambda t: t.float().numpy().astype(np.float64)
    res = {}

    # B=1, T=1024 gated local layer (the small check workload), in full
    x = si.prefill_layer(si.generator(1000), 1, 1024, HQ, HKV, D, gated=True)
    t0 = time.perf_counter()
    oracle.prefill(f(x["q"]), f(x["k"]), f(x["v"]), f(x["gate"]), window=W, gated=True,
                   rope_base=1e4)
    dt = time.perf_counter() - t0
    res["t1024_local"] = {"value": round(1024 / dt, 1), "unit": "tokens/s", "cores": cores,
                          "kind": "oracle", "sample": "the whole layer (B=1, T=1024, W=128, gated)",
                          "seconds": round(dt, 2)}
    log(f"[bench] oracle T=1024 local layer: {dt:.2f} s")

    # B=64 decode step: the ring (local) step in full; the linear (global) step on sequences drawn
    # from the same length distribution until about budget_s seconds, scaled to the 64
    rng = np.random.default_rng(1002)
    Bd, lo, hi = 64, 8192, 65536
    lens = rng.integers(lo, hi + 1, Bd)
    qn, kn, vn, g = (rng.standard_normal(s_) for s_ in
                     ((Bd, HQ, D), (Bd, HKV, D), (Bd, HKV, D), (Bd, HQ, D)))
    kr, vr = rng.standard_normal((Bd, W, HKV, D)), rng.standard_normal((Bd, W, HKV, D))
    t0 = time.perf_counter()
    oracle.decode(qn, kn, vn, g, kr, vr, lens, window=W, gated=True, rope_base=1e7)
    t_ring = time.perf_counter() - t0
    done, t_lin = 0, 0.0
    while done < Bd and t_lin < budget_s:
        L = int(lens[done])
        kc = rng.standard_normal((1, L, HKV, D))
        vc = rng.standard_normal((1, L, HKV, D))
        t0 = time.perf_counter()
        oracle.decode(qn[done:done + 1], kn[done:done + 1], vn[done:done + 1], None, kc, vc,
                      lens[done:done + 1], window=0, gated=False, rope_base=1e7)
        t_lin += time.perf_counter() - t0
        done += 1
        del kc, vc
    t_lin_step = t_lin / float(lens[:done].sum()) * float(lens.sum())
    res["decode_b64"] = {
        "ring": {"value": round(Bd / t_ring, 1), "unit": "tokens/s", "cores": cores,
                 "kind": "oracle", "sample": "the whole B=64 ring step", "seconds": round(t_ring, 3)},
        "linear": {"value": round(Bd / t_lin_step, 2), "unit": "tokens/s", "cores": cores,
                   "kind": "oracle",
                   "sample": f"{done} of the 64 sequences ({int(lens[:done].sum())} keys), step time "
                             f"scaled by total keys (extrapolated)",
                   "seconds_sampled": round(t_lin, 2), "step_seconds_extrapolated": round(t_lin_step, 1)}}
    log(f"[bench] oracle decode: ring step {t_ring:.3f} s, linear step {t_lin_step:.1f} s (extrapolated)")

    # B=1, T=262144 layer pair: local rows at uniform positions; global rows near the middle in
    # one call (the prologue over the keys is shared by the rows of a call)
    Tl = 262144
    q = rng.standard_normal((1, Tl, HQ, D), dtype=np.float32)
    k = rng.standard_normal((1, Tl, HKV, D), dtype=np.float32)
    v = rng.standard_normal((1, Tl, HKV, D), dtype=np.float32)
    rows_l = np.sort(rng.integers(W, Tl, 128))
    t0 = time.perf_counter()
    for r_ in rows_l:  # one call per row: a call normalises every key between its first and last row
        oracle.prefill_rows(q, k, v, q, [r_], window=W, gated=True, rope_base=1e7)
    t_l = (time.perf_counter() - t0) / len(rows_l)
    mid = Tl // 2
    rows_g = [mid - 3, mid - 2, mid - 1, mid]
    t0 = time.perf_counter()
    oracle.prefill_rows(q, k, v, None, rows_g, window=0, gated=False, rope_base=1e7)
    t_call = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.prefill_rows(q, k, v, None, rows_g[-1:], window=0, gated=False, rope_base=1e7)
    t_one = time.perf_counter() - t0
    t_row_mid = max((t_call - t_one) / 3.0, 1e-9)       # one more row at the mean position
    t_shared = max(t_one - t_row_mid, 0.0)               # key prologue of half the sequence
    t_glob = 2 * t_shared + Tl * t_row_mid               # whole layer, extrapolated
    del q, k, v
    res["t262144"] = {
        "local": {"value": round(1.0 / t_l, 1), "unit": "tokens/s", "cores": cores,
                  "kind": "oracle", "sample": f"{len(rows_l)} rows at uniform positions, one call each",
                  "layer_seconds_extrapolated": round(Tl * t_l, 1)},
        "global": {"value": round(Tl / t_glob, 3), "unit": "tokens/s", "cores": cores,
                   "kind": "oracle",
                   "sample": "rows at T/2 (the mean causal row): one row, then four in one call; "
                             "layer time = key prologue + T x per-row time (extrapolated)",
                   "layer_seconds_extrapolated": round(t_glob, 1)}}
    log(f"[bench] oracle T=262144: local {t_l * 1e3:.2f} ms/row, global layer ~{t_glob:.0f} s")

    # one teacher-forced layer of the 32-layer stack (T=65536, hidden 4096): sampled rows; the k/v
    # projections of the rows' keys are shared by the rows of a call
    Ts, hidden = 65536, 4096
    xs = rng.standard_normal((Ts, hidden))
    wts = {n_: rng.standard_normal(s_) * 0.02 for n_, s_ in
           (("wq", (HQ * D, hidden)), ("wk", (HKV * D, hidden)), ("wv", (HKV * D, hidden)),
            ("wg", (HQ * D, hidden)), ("wo", (hidden, HQ * D)))}
    rows = np.sort(rng.integers(W, Ts, 32))
    t0 = time.perf_counter()
    oracle.stack_layer_rows(xs, wts, rows, is_global=False, rope_base=1e7)
    t_loc = (time.perf_counter() - t0) / len(rows)
    mid = Ts // 2
    t0 = time.perf_counter()
    oracle.stack_layer_rows(xs, wts, [mid], is_global=True, rope_base=1e7)
    t_g1 = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.stack_layer_rows(xs, wts, [mid - 3, mid - 2, mid - 1, mid], is_global=True, rope_base=1e7)
    t_g4 = time.perf_counter() - t0
    t_grow = max((t_g4 - t_g1) / 3.0, 1e-9)
    t_gshared = max(t_g1 - t_grow, 0.0)                  # k/v projections of half the keys
    t_glayer = 2 * t_gshared + Ts * t_grow
    t_stack = 27 * Ts * t_loc + 5 * t_glayer
    del xs, wts
    res["stack_t65536"] = {
        "value": round(Ts / t_stack, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
        "sample": f"teacher-forced layers on host-drawn inputs: {len(rows)} local rows; global rows at "
                  f"T/2 (one, then four in one call); 32-layer time = 27 local layers at the per-row "
                  f"time + 5 global layers at (shared k/v projection + T x per-row time) "
                  f"(extrapolated)",
        "local_ms_per_row": round(t_loc * 1e3, 2), "global_layer_seconds_extrapolated": round(t_glayer, 1),
        "stack_seconds_extrapolated": round(t_stack, 1)}
    log(f"[bench] oracle stack: local {t_loc * 1e3:.1f} ms/row, global layer ~{t_glayer:.0f} s")
    return res


def cpu_baseline(torch, si, budget_s=12.0):
    """The fp64 oracle on the host cores, on a bounded sample of the same 5:1 block: query rows of
    sequence 0 (all 32 heads) of a gated local layer and of the global layer, drawn at uniform
    positions and processed in batches until about budget_s seconds of CPU work are spent (40%
    local, 60% global). Rate = tokens/s of a 5:1 block = 1 / (5 * t_row_local + t_row_global),
    with the global row time scaled to the mean position of a full sequence."""
    import numpy as np
    import oracle
    threads = _oracle_threads()
    gen = si.generator(SEED)
    Ts = 16384
    x = si.prefill_layer(gen, 1, Ts, HQ, HKV, D, gated=True)
    f = lambda t: t.float().numpy().astype(np.float64)
    q, k, v, g = f(x["q"]), f(x["k"]), f(x["v"]), f(x["gate"])
    rng = np.random.default_rng(0)
    order_l = rng.permutation(np.arange(W, Ts))
    order_g = rng.permutation(np.arange(Ts))

    def timed(order, batch, budget, **kw):
        n, t0 = 0, time.perf_counter()
        while n < len(order) and time.perf_counter() - t0 < budget:
            rows = np.sort(order[n:n + batch])
            oracle.prefill_rows(q, k, v, g if kw["gated"] else None, rows, rope_base=ROPE_BASE, **kw)
            n += len(rows)
        return n, time.perf_counter() - t0, order[:n]

    n_l, t_l, _ = timed(order_l, 64, 0.4 * budget_s, window=W, gated=True)
    n_g, t_g, rows_g = timed(order_g, 16, 0.6 * budget_s, window=0, gated=False)
    t_row_l = t_l / n_l
    t_row_g = t_g / n_g * ((Ts + 1) / 2) / float(np.mean(rows_g + 1))
    rate = 1.0 / (5 * t_row_l + t_row_g)
    log(f"[bench] oracle: {t_row_l * 1e3:.2f} ms/local row ({n_l} rows), "
        f"{t_row_g * 1e3:.2f} ms/global row ({n_g} rows)")
    return {"value": round(rate, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_l} local-layer rows + {n_g} global-layer rows of sequence 0 (all 32 "
                      f"heads), T={Ts}, uniform positions; global row time scaled to the mean "
                      f"position; {t_l + t_g:.1f} s of CPU work"}


if __name__ == "__main__":
    main()
