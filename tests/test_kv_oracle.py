"""KV sizing and layer schedule of the oracle against the figures printed on the pages."""
import json
import os

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kv_footprint.json")))
UNIT = {"KiB": 2 ** 10, "GiB": 2 ** 30}


def _kv(fn, global_every, T, n_layers=32, batch=1):
    return fn(n_layers, global_every, GOLD["n_kv_heads"], GOLD["head_dim"], GOLD["window"],
              GOLD["elem_bytes"], batch, T)


def check_kv_function(fn):
    """Shared by the oracle test here and by the C ABI test: every printed figure must match."""
    e = {x["what"]: x for x in GOLD["entries"]}
    for what in ("per-token KV, all 32 layers global", "per-token KV, hybrid 5 global + 27 SWA"):
        x = e[what]
        slope = _kv(fn, x["global_every"], 200000) - _kv(fn, x["global_every"], 199999)
        assert slope == x["value"] * UNIT[x["unit"]], what
    for what in ("KV at 256K context, all global", "KV at 256K context, hybrid"):
        x = e[what]
        b = _kv(fn, x["global_every"], x["seqlen"], batch=x["batch"])
        assert round(b / UNIT[x["unit"]], x["decimals"]) == x["value"], (what, b)
    full = _kv(fn, 1, 262144)
    hyb = _kv(fn, 6, 262144)
    assert full == 34359738368                         # exactly 32 GiB
    assert hyb == 5 * 262144 * 4096 + 27 * 128 * 4096   # exact, includes the 27 rings
    assert round(full / hyb, 1) == e["reduction all-global / hybrid"]["value"]
    slope_full = _kv(fn, 1, 10 ** 6) - _kv(fn, 1, 10 ** 6 - 1)
    slope_hyb = _kv(fn, 6, 10 ** 6) - _kv(fn, 6, 10 ** 6 - 1)
    assert slope_full / slope_hyb == 6.4
    gd = GOLD["gdn_comparison"]
    gdn = _kv(fn, 1, 262144, n_layers=gd["global_layers"])
    assert round(gdn / UNIT[gd["unit"]], gd["decimals"]) == gd["value"]
    # below the window every layer stores every token
    assert _kv(fn, 6, 100) == _kv(fn, 1, 100)
    assert _kv(fn, 6, 0) == 0
    assert _kv(fn, 6, 5, batch=3) == 3 * _kv(fn, 6, 5)


def test_oracle_kv_bytes():
    check_kv_function(oracle.kv_bytes)


def test_toy_entry_count():
    t = GOLD["toy"]
    assert oracle.kv_entries(t["n_layers"], t["global_every"], t["window"], t["seqlen"]) == t["hybrid_entries"]
    assert oracle.kv_entries(t["n_layers"], 1, t["window"], t["seqlen"]) == t["full_entries"]


def test_layer_schedule():
    s = GOLD["schedule"]
    gl = oracle.global_layers(32, 6)
    assert gl == s["global_layers_1based"]
    assert gl[-1] - 1 == s["last_global_0based"]
    assert 32 - gl[-1] == s["trailing_swa"]
    assert len(gl) == 5 and 32 - len(gl) == 27
