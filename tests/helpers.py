"""Shared test utilities: tensor conversion and the bf16 parity bar.

Parity bar for bf16 outputs (fp32 accumulation on the GPU, fp64 oracle): max-abs error <= 2e-2 and
mean-abs error <= 2e-3 over the compared elements.
"""
import numpy as np
import torch

MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").float().numpy().astype(np.float64)


def err_stats(got, ref):
    got = f64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    e = np.abs(got - ref)
    rel_rms = float(np.sqrt(np.mean(e ** 2)) / max(np.sqrt(np.mean(ref ** 2)), 1e-30))
    return float(e.max()), float(e.mean()), rel_rms


def assert_parity(got, ref, what="", max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    mx, mean, rel = err_stats(got, ref)
    print(f"[parity] {what}: max_abs={mx:.3e} mean_abs={mean:.3e} rel_rms={rel:.3e}", flush=True)
    assert np.isfinite(mx), f"{what}: non-finite output"
    assert mx <= max_abs, f"{what}: max abs err {mx:.3e} > {max_abs}"
    assert mean <= mean_abs, f"{what}: mean abs err {mean:.3e} > {mean_abs}"
    return mx, mean, rel
