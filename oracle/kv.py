"""Integer oracle of KV-cache sizing and of the 5:1 layer schedule. TEST INFRASTRUCTURE ONLY.

ZGCM-1 zh-TW translation page §2.1 "Model overview": 32 layers, 27 gated-SWA layers with a 128-token
window and 5 global causal layers at layers 6, 12, 18, 24, 30 (five blocks of five local layers and one
global layer, then two trailing local layers). §2.3 "KV cache analysis": SWA layers keep only a fixed
128-token window in the KV cache and global layers keep the whole sequence.

Parity pins (tests/test_kv_oracle.py): the pages' closed forms -- 128 KiB vs 20 KiB per token, 32.0 GiB
vs 5.0 GiB at 256K (6.4x), 7.0 GiB for the GDN 3:1 comparison (Fig. 4c of the English explainer page),
and the explainer's toy count of 24 vs 40 KV entries (window 4, 8 tokens, 4 local + 1 global layers);
the layer list 6/12/18/24/30 and "last global layer is 29 (0-indexed)" (English explainer, Fig. 3).
"""
from __future__ import annotations


def is_global_layer(layer_1based: int, global_every: int) -> bool:
    """Layer l (1-indexed) is global iff global_every > 0 and l is a multiple of global_every."""
    return global_every > 0 and layer_1based % global_every == 0


def global_layers(n_layers: int, global_every: int) -> list[int]:
    """1-indexed global layers of an n-layer stack."""
    return [l for l in range(1, n_layers + 1) if is_global_layer(l, global_every)]


def kv_entries(n_layers: int, global_every: int, window: int, seqlen: int) -> int:
    """Cached token entries per sequence and per KV head: a global layer stores every position, a
    local layer stores at most `window` of them (window <= 0 means the layer stores all)."""
    total = 0
    for l in range(1, n_layers + 1):
        if is_global_layer(l, global_every) or window <= 0:
            total += seqlen
        else:
            total += min(seqlen, window)
    return total


def kv_bytes(n_layers: int, global_every: int, n_kv_heads: int, head_dim: int, window: int,
             elem_bytes: int, batch: int, seqlen: int) -> int:
    """Exact bytes of K and V caches: entries x 2 (K and V) x heads x head_dim x element size x
    batch."""
    return kv_entries(n_layers, global_every, window, seqlen) * 2 * n_kv_heads * head_dim \
        * elem_bytes * batch
