"""Seeded synthetic inputs for the hybrid attention core: the only module the GPU tests, bench.py and
the oracle checks share. It draws random numbers and lays them out; it holds none of the attention
arithmetic.

Every tensor is drawn as float32 N(0, std^2) from a seeded torch generator and rounded (RNE) to
bfloat16, so the GPU path and the oracle consume identical bf16 values (the oracle widens them to
fp64). Seed convention: 1000 + the index of the workload in the fixed list of five workloads
(T=1024 check, B=4 x 16K prefill pair, B=64 decode step, 256K prefill pair, 32-layer stack).
"""
from __future__ import annotations

import torch

SEED_BASE = 1000


def generator(seed: int, device="cpu") -> torch.Generator:
    return torch.Generator(device=device).manual_seed(int(seed))


def randn_bf16(gen: torch.Generator, shape, std: float = 1.0, device="cpu") -> torch.Tensor:
    x = torch.randn(tuple(shape), generator=gen, dtype=torch.float32, device=device)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def prefill_layer(gen, B, T, Hq=32, Hkv=8, D=128, gated=True, device="cpu"):
    """q, k, v and (for gated layers) gate logits, in that draw order. q/gate: [B,T,Hq,D],
    k/v: [B,T,Hkv,D]."""
    q = randn_bf16(gen, (B, T, Hq, D), device=device)
    k = randn_bf16(gen, (B, T, Hkv, D), device=device)
    v = randn_bf16(gen, (B, T, Hkv, D), device=device)
    g = randn_bf16(gen, (B, T, Hq, D), device=device) if gated else None
    return {"q": q, "k": k, "v": v, "gate": g}


def seqlens_uniform(gen, B, lo, hi, device="cpu") -> torch.Tensor:
    """Context lengths uniform on the integers [lo, hi] (int32)."""
    return torch.randint(lo, hi + 1, (B,), generator=gen, device=device, dtype=torch.int64) \
        .to(torch.int32)


def decode_step(gen, B=64, Hq=32, Hkv=8, D=128, window=128, len_lo=8192, len_hi=65536,
                cache_stride=None, device="cpu"):
    """One decode step for a local and a global layer, draw order: seqlens, ring K, ring V,
    linear K, linear V (rows < seqlens[b]-1 only; the rest stay zero), q_new, k_new, v_new, gate.
    Cache contents stand for already normalised and rotated keys; they are N(0,1) like every
    other input."""
    seqlens = seqlens_uniform(gen, B, len_lo, len_hi, device=device)
    stride = int(cache_stride or len_hi)
    ring_k = randn_bf16(gen, (B, window, Hkv, D), device=device)
    ring_v = randn_bf16(gen, (B, window, Hkv, D), device=device)
    lin_k = torch.zeros((B, stride, Hkv, D), dtype=torch.bfloat16, device=device)
    lin_v = torch.zeros((B, stride, Hkv, D), dtype=torch.bfloat16, device=device)
    lens = seqlens.tolist()
    for b in range(B):
        n = lens[b] - 1
        lin_k[b, :n] = randn_bf16(gen, (n, Hkv, D), device=device)
    for b in range(B):
        n = lens[b] - 1
        lin_v[b, :n] = randn_bf16(gen, (n, Hkv, D), device=device)
    q_new = randn_bf16(gen, (B, Hq, D), device=device)
    k_new = randn_bf16(gen, (B, Hkv, D), device=device)
    v_new = randn_bf16(gen, (B, Hkv, D), device=device)
    gate = randn_bf16(gen, (B, Hq, D), device=device)
    return {"seqlens": seqlens, "ring_k": ring_k, "ring_v": ring_v, "lin_k": lin_k,
            "lin_v": lin_v, "q_new": q_new, "k_new": k_new, "v_new": v_new, "gate": gate,
            "cache_stride": stride}


def stack_layer_weights(gen, hidden=4096, Hq=32, Hkv=8, D=128, is_global=False, std=0.02,
                        device="cpu"):
    """[out, in] bf16 weights of one attention layer, draw order wq, wk, wv, (wg), wo."""
    w = {"wq": randn_bf16(gen, (Hq * D, hidden), std, device),
         "wk": randn_bf16(gen, (Hkv * D, hidden), std, device),
         "wv": randn_bf16(gen, (Hkv * D, hidden), std, device)}
    if not is_global:
        w["wg"] = randn_bf16(gen, (Hq * D, hidden), std, device)
    w["wo"] = randn_bf16(gen, (hidden, Hq * D), std, device)
    return w


def stack_input(gen, B, T, hidden=4096, device="cpu") -> torch.Tensor:
    """Residual-stream input x0 ~ N(0,1), kept in float32 (drawn as bf16 values)."""
    return randn_bf16(gen, (B, T, hidden), device=device).float()


def ramped_logits_layer(gen, T, Hq=32, Hkv=8, D=128, window=0, noise=0.05, period=96,
                        device="cpu"):
    """Inputs whose attention scores sweep a wide range smoothly along the key axis (for the
    running-reference rescale path of the kernels; used with a q norm weight of a few units).

    Two fixed directions u and w, nonzero only on dims >= 42 (the unrotated ones) and of unit RMS
    over D, with w orthogonal to u. q rows are u + noise; key j is cos(th_j) u + sin(th_j) w + noise
    with th_j falling from pi to 0 over the sequence (window 0) or over every `period` keys (a
    sawtooth, window > 0); v is a smooth function of the position, sin(2 pi j / 200 + d / 7 + kv
    head); gate logits are N(0, 1). Draw order: u, w, q noise, k noise, gate."""
    u = torch.zeros(D)
    u[42:] = torch.randn(D - 42, generator=gen)
    w = torch.zeros(D)
    w[42:] = torch.randn(D - 42, generator=gen)
    u = u.double()
    w = w.double()
    w = w - (w @ u) / (u @ u) * u
    u = u / torch.sqrt(torch.mean(u * u))
    w = w / torch.sqrt(torch.mean(w * w))
    j = torch.arange(T, dtype=torch.float64)
    frac = j / max(T - 1, 1) if window == 0 else (j % period) / (period - 1)
    th = torch.pi * (1.0 - frac)
    q = u + noise * torch.randn((T, Hq, D), generator=gen).double()
    k = (torch.cos(th)[:, None, None] * u + torch.sin(th)[:, None, None] * w
         + noise * torch.randn((T, Hkv, D), generator=gen).double())
    d = torch.arange(D, dtype=torch.float64)
    h = torch.arange(Hkv, dtype=torch.float64)
    v = torch.sin(2 * torch.pi * j[:, None, None] / 200.0 + d / 7.0 + h[:, None])
    g = torch.randn((T, Hq, D), generator=gen).double()
    to = lambda a: a.float().to(torch.bfloat16)[None].to(device)
    return {"q": to(q), "k": to(k), "v": to(v), "gate": to(g)}
