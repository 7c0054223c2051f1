"""Host-side checks of the C ABI that need no GPU: the library loads, exports every function the
header declares, sizes KV caches to the pages' figures, and rejects bad arguments before any launch."""
import ctypes
import os
import re

import pytest

import global_causal_attention_amd as zg
from global_causal_attention_amd._abi import ZgAttnCfg

from test_kv_oracle import check_kv_function

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "zg_attn.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(zg_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(zg.LIB_PATH)
    names = _declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(zg.EXPORTS), "ctypes table and header disagree"


def test_kv_bytes_matches_pages():
    check_kv_function(zg.zg_kv_bytes)


def test_kv_bytes_rejects_negative():
    with pytest.raises(zg.ZGError):
        zg.zg_kv_bytes(32, 6, 8, 128, 128, 2, -1, 10)


def _call_prefill(cfg, B=1, T=4, q=16, k=16, v=16, gate=16, out=16, ws=256, ws_bytes=1 << 20):
    lib = zg.load_library()
    c = cfg.c() if cfg is not None else None
    return lib.zg_attn_prefill(ctypes.byref(c) if c is not None else None, B, T, 0, q, k, v, gate,
                               None, None, None, out, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), zg.ZG_ERR_UNSUPPORTED),
    (dict(n_q_heads=12, n_kv_heads=1), zg.ZG_ERR_UNSUPPORTED),
    (dict(n_q_heads=32, n_kv_heads=6), zg.ZG_ERR_SHAPE),
    (dict(rot_dim=43), zg.ZG_ERR_UNSUPPORTED),
    (dict(rot_dim=66), zg.ZG_ERR_UNSUPPORTED),
    (dict(window=-1), zg.ZG_ERR_SHAPE),
    (dict(rope_base=1.0), zg.ZG_ERR_SHAPE),
    (dict(rms_eps=-1.0), zg.ZG_ERR_SHAPE),
])
def test_prefill_rejects_bad_config(kw, status):
    assert _call_prefill(zg.AttnConfig(**kw)) == status
    assert zg.zg_last_error() != ""


def test_prefill_rejects_bad_arguments():
    cfg = zg.AttnConfig()
    lib = zg.load_library()
    assert lib.zg_attn_prefill(None, 1, 4, 0, 16, 16, 16, 16, None, None, None, 16, 256, 1 << 20,
                               None) == zg.ZG_ERR_NULL
    assert _call_prefill(cfg, q=None) == zg.ZG_ERR_NULL
    assert _call_prefill(cfg, gate=None) == zg.ZG_ERR_NULL
    assert _call_prefill(cfg, B=0) == zg.ZG_ERR_SHAPE
    assert _call_prefill(cfg, T=0) == zg.ZG_ERR_SHAPE
    assert _call_prefill(cfg, q=8) == zg.ZG_ERR_SHAPE            # misaligned
    assert _call_prefill(cfg, ws=None) == zg.ZG_ERR_WORKSPACE
    assert _call_prefill(cfg, ws_bytes=10) == zg.ZG_ERR_WORKSPACE
    need = zg.zg_attn_prefill_workspace_bytes(cfg, 2, 100)
    assert need >= 2 * 100 * 8 * 128 * 2


def test_decode_rejects_bad_arguments():
    lib = zg.load_library()
    cfg = zg.AttnConfig(window=0, gated=False)
    c = cfg.c()
    ws = zg.zg_attn_decode_workspace_bytes(cfg, 4, 100000)
    assert ws >= 4 * 32 * 128 * 4

    def call(B=4, stride=100000, max_len=100000, ws_bytes=ws, seq=16):
        return lib.zg_attn_decode(ctypes.byref(c), B, stride, max_len, 16, 16, 16, None, None, None,
                                  16, 16, seq, 16, 256, ws_bytes, None)
    assert call(stride=10) == zg.ZG_ERR_SHAPE
    assert call(max_len=0) == zg.ZG_ERR_SHAPE
    assert call(B=0) == zg.ZG_ERR_SHAPE
    assert call(ws_bytes=ws - 1) == zg.ZG_ERR_WORKSPACE
    assert call(seq=None) == zg.ZG_ERR_NULL


def test_gemm_and_rmsnorm_reject_bad_arguments():
    lib = zg.load_library()
    assert lib.zg_gemm_bf16(16, 64, 100, 16, 16, None, 16, 64, None) == zg.ZG_ERR_SHAPE
    assert lib.zg_gemm_bf16(16, 64, 128, 16, 16, None, None, 64, None) == zg.ZG_ERR_NULL
    assert lib.zg_gemm_bf16(16, 64, 128, 16, 16, None, 16, 32, None) == zg.ZG_ERR_SHAPE
    assert lib.zg_rmsnorm(4, 12, 16, None, 1e-6, 16, None) == zg.ZG_ERR_SHAPE
    assert lib.zg_rmsnorm(4, 128, None, None, 1e-6, 16, None) == zg.ZG_ERR_NULL


def test_prefill_cached_rejects_bad_arguments():
    lib = zg.load_library()
    c = zg.AttnConfig(window=0, gated=False).c()
    ws = 256
    # linear cache shorter than pos0 + T
    st = lib.zg_attn_prefill_cached(ctypes.byref(c), 1, 8, 100, 16, 16, 16, None, None, None, None,
                                    16, 16, 100, 16, ws, 1 << 20, None)
    assert st == zg.ZG_ERR_SHAPE
    # missing cache
    st = lib.zg_attn_prefill_cached(ctypes.byref(c), 1, 8, 0, 16, 16, 16, None, None, None, None,
                                    None, 16, 100, 16, ws, 1 << 20, None)
    assert st == zg.ZG_ERR_NULL
    # ring caches need the staging workspace
    cr = zg.AttnConfig(window=128, gated=False).c()
    assert zg.zg_attn_prefill_cached_workspace_bytes(zg.AttnConfig(window=128, gated=False), 1, 8) > 0
    assert zg.zg_attn_prefill_cached_workspace_bytes(zg.AttnConfig(window=0, gated=False), 1, 8) == 0
    st = lib.zg_attn_prefill_cached(ctypes.byref(cr), 1, 8, 0, 16, 16, 16, None, None, None, None,
                                    16, 16, 0, 16, None, 0, None)
    assert st == zg.ZG_ERR_WORKSPACE


def test_training_entry_points_reject_bad_arguments():
    lib = zg.load_library()
    c = zg.AttnConfig(window=128, gated=True).c()
    # the training kernels take 4 query heads per KV head only
    c8 = zg.AttnConfig(n_q_heads=8, n_kv_heads=1, window=0, gated=False).c()
    st = lib.zg_attn_forward_train(ctypes.byref(c8), 1, 8, 16, 16, 16, None, 16, 16, 16, 1 << 20, None)
    assert st == zg.ZG_ERR_UNSUPPORTED
    # gated without a gate
    st = lib.zg_attn_forward_train(ctypes.byref(c), 1, 8, 16, 16, 16, None, 16, 16, 16, 1 << 20, None)
    assert st == zg.ZG_ERR_NULL
    # missing lse
    st = lib.zg_attn_backward(ctypes.byref(c), 1, 8, 16, 16, 16, 16, 16, 16, None, 16, 16, 16, 16,
                              16, 1 << 30, None)
    assert st == zg.ZG_ERR_NULL
    # workspace too small
    need = lib.zg_attn_backward_workspace_bytes(ctypes.byref(c), 1, 8)
    assert need > 0
    st = lib.zg_attn_backward(ctypes.byref(c), 1, 8, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16,
                              16, need - 1, None)
    assert st == zg.ZG_ERR_WORKSPACE
    st = lib.zg_attn_backward(ctypes.byref(c), 0, 8, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16,
                              16, need, None)
    assert st == zg.ZG_ERR_SHAPE


def test_read_probe_rejects_bad_arguments():
    lib = zg.load_library()
    assert lib.zg_hbm_read_probe(None, 1024, 16, 4, None) == zg.ZG_ERR_NULL
    assert lib.zg_hbm_read_probe(16, 1000, 16, 4, None) == zg.ZG_ERR_SHAPE
    assert lib.zg_hbm_read_probe(16, 1024, 16, 0, None) == zg.ZG_ERR_SHAPE
    assert lib.zg_hbm_read_probe(8, 1024, 16, 4, None) == zg.ZG_ERR_SHAPE


def test_decode_key_limit_matches_header():
    """The header allows at most 2^21 = 2,097,152 keys per sequence (linear max_seqlen); one more
    is UNSUPPORTED. At the limit the call gets past that check and stops at the (too small)
    workspace, before any launch."""
    lib = zg.load_library()
    limit = 1 << 21
    assert "2^21" in open(HEADER).read()
    for fp8 in (False, True):
        cfg = zg.AttnConfig(window=0, gated=False)
        c = cfg.c()
        need = zg.zg_attn_decode_workspace_bytes(cfg, 1, limit)

        def call(max_len):
            args = (ctypes.byref(c), 1, max_len, max_len, 16, 16, 16, None, None, None, 16, 16)
            tail = (16, 16, 256, need - 16, None)
            if fp8:
                return lib.zg_attn_decode_fp8(*args, ctypes.c_float(1.0), ctypes.c_float(1.0), *tail)
            return lib.zg_attn_decode(*args, *tail)
        assert call(limit + 1) == zg.ZG_ERR_UNSUPPORTED, zg.zg_last_error()
        assert call(limit) == zg.ZG_ERR_WORKSPACE, zg.zg_last_error()


def test_decode_noalloc_rejects_before_touching_the_device():
    """zg_attn_decode_noalloc checks every argument and its 96 MiB scratch limit before it looks
    up the scratch address or launches anything (these calls run without a GPU)."""
    lib = zg.load_library()
    c = zg.AttnConfig(window=0, gated=False).c()

    def call(B=64, stride=200000, max_len=200000, seq=16, q=16):
        return lib.zg_attn_decode_noalloc(ctypes.byref(c), B, stride, max_len, q, 16, 16, None,
                                          None, None, 16, 16, seq, 16, None)
    assert call(q=None) == zg.ZG_ERR_NULL
    assert call(seq=None) == zg.ZG_ERR_NULL
    assert call(B=0) == zg.ZG_ERR_SHAPE
    assert call(stride=10) == zg.ZG_ERR_SHAPE
    # B = 64 sequences of up to 200,000 keys need ~213 MB of partials: beyond the static scratch
    assert call() == zg.ZG_ERR_UNSUPPORTED
    assert "96" in zg.zg_last_error() or "scratch" in zg.zg_last_error()
    assert zg.zg_attn_decode_workspace_bytes(zg.AttnConfig(window=0, gated=False), 64, 94208) \
        <= 96 << 20
    assert zg.zg_attn_decode_workspace_bytes(zg.AttnConfig(window=0, gated=False), 64, 94209) \
        > 96 << 20


def test_forward_train_workspace_query():
    """The training forward runs the tiled kernel on keys normalised and rotated into its
    workspace: B T Hkv 256 bytes (rounded up to 256), then 2 KB of item counters for the
    attention launch; a smaller workspace is rejected before any launch."""
    band = zg.AttnConfig(window=128, gated=True)
    assert zg.zg_attn_forward_train_workspace_bytes(band, 2, 1000) == 2 * 1000 * 8 * 256 + 2048
    lib = zg.load_library()
    c = band.c()
    need = zg.zg_attn_forward_train_workspace_bytes(band, 1, 1000)
    st = lib.zg_attn_forward_train(ctypes.byref(c), 1, 1000, 16, 16, 16, 16, 16, 16, 16, need - 16,
                                   None)
    assert st == zg.ZG_ERR_WORKSPACE
