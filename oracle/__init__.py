"""fp64 CPU oracle of the ZGCM-1 hybrid attention core. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this package. The GPU library never calls it and it never imports the GPU library: the two share no
code. Every function takes plain NumPy arrays (the exact fp64 widening of the bf16 inputs) and
evaluates the plain definition of what the hot path computes, with no tiling, no online softmax and no
rounding of intermediates.

Sources (all pages describe one paper, "ZGCM-1: A Fully Open and Extremely Efficient Foundation Model
for Math and Agentic Search"):

* zh-TW translation page (papers.lianghsun.dev): §2.1 "Model overview" and Fig. 3 (layer schedule,
  gated SWA formula, QK-RMSNorm, partial RoPE with rotary fraction 0.33); §2.3 "KV cache analysis"
  (per-token and 256K footprints); §3.2 "Mid-training" (RoPE base 10M at 256K).
* zh-CN tutorial page (agifrontier.github.io): the architecture paragraph (same formula and numbers).
* English explainer page (paperglide.net): Fig. 3 and Fig. 4 captions, and the toy KV-entry count
  (window 4, 8 tokens, 4 SWA + 1 global layers: 24 vs 40 entries).
* FP8: the E4M3 format the pages train their forward matrix multiplications in (zh-TW page §3.1,
  hyper-parameters), used here for the decode KV cache (``fp8.py``) and the layer's projections
  (``fp8_stack.py``).

Parity status per function is listed in each module's header.
"""
from .attention import (rms_norm, rope_inv_freq, partial_rope, qk_prologue, key_set,
                        prefill, prefill_rows, attention_probs_row, decode)
from .kv import kv_bytes, kv_entries, is_global_layer, global_layers
from .stack import stack_layer, stack_layer_rows, stack, layer_is_global
from .fp8 import e4m3_values, round_e4m3, decode_fp8_cache
from .backward import layer_backward, layer_backward_rows, row_lse
from .fp8_stack import (e4m3_decode, quant_rows_e4m3, gemm_e4m3, quantize_layer_weights,
                        stack_layer_fp8, stack_layer_rows_fp8, stack_fp8)

__all__ = [
    "rms_norm", "rope_inv_freq", "partial_rope", "qk_prologue", "key_set", "prefill",
    "prefill_rows", "attention_probs_row", "decode", "kv_bytes", "kv_entries",
    "is_global_layer", "global_layers", "stack_layer", "stack_layer_rows", "stack", "layer_is_global",
    "e4m3_values", "round_e4m3", "decode_fp8_cache", "layer_backward", "layer_backward_rows",
    "row_lse", "e4m3_decode", "quant_rows_e4m3", "gemm_e4m3", "quantize_layer_weights",
    "stack_layer_fp8", "stack_layer_rows_fp8", "stack_fp8",
]
