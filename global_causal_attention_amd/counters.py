"""Summaries of rocprofv3 output for profiles/, and the lookup bench.py uses for HBM traffic.

Kernel-time summary (from the kernel trace of `rocprofv3 --kernel-trace --stats --output-format
csv`, per kernel and grid size):
    python -m global_causal_attention_amd.counters stats <run_kernel_trace.csv> <out.md> -- <cmd..>

HBM traffic per dispatch (from two `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of the
same command; both counters are in KiB per dispatch). Each counter is scaled by the ratio between
the true bytes of a plain device copy of known size in the same run and what the counter reads for
it, so the figures are HBM bytes:
    python -m global_causal_attention_amd.counters traffic <fetch.csv> <write.csv> <copy_bytes> \
        <out.json> <out.md> -- <cmd..>

SQ counter summary (from one or more `rocprofv3 --pmc <counters>` runs):
    python -m global_causal_attention_amd.counters util <counter_collection.csv>... <out.md> -- <cmd..>

The JSON records, per kernel, the sha256 of the sources that build it; `lookup_traffic` returns
None once those sources differ from the ones the counters were taken with.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_JSON = os.path.join(PROFILES, "hbm_traffic.json")
COPY_KERNEL = "__amd_rocclr_copyBuffer"

# sources that determine each kernel's code (shared headers included)
_CSRC = os.path.join(PKG, "csrc")
_COMMON = ["zg_common.hpp", "zg_kernels.hpp", "zg_mfma.hpp"]
KERNEL_SOURCES = {
    "kprep_kernel": ["prefill.hip"] + _COMMON,
    "prefill_kernel": ["prefill.hip"] + _COMMON,
    "prefill_swa_kernel": ["prefill_swa.hip"] + _COMMON,
    "decode_prep_kernel": ["decode.hip"] + _COMMON,
    "decode_attn_kernel": ["decode.hip"] + _COMMON,
    "decode_attn_fp8_kernel": ["decode.hip"] + _COMMON,
    "decode_mfma_kernel": ["decode.hip"] + _COMMON,
    "bwd_pre_kernel": ["backward.hip"] + _COMMON,
    "bwd_q_kernel": ["backward.hip"] + _COMMON,
    "bwd_kv_kernel": ["backward.hip"] + _COMMON,
    "decode_combine_kernel": ["decode.hip"] + _COMMON,
    "decode_ring_kernel": ["decode.hip"] + _COMMON,
    "row_copy_kernel": ["prefill.hip"] + _COMMON,
    "rmsnorm_kernel": ["stack.hip"] + _COMMON,
    "gemm_kernel": ["stack.hip"] + _COMMON,
    "rmsnorm_fp8_kernel": ["stack_fp8.hip"] + _COMMON,
    "quant_rows_kernel": ["stack_fp8.hip"] + _COMMON,
    "gemm_fp8_kernel": ["stack_fp8.hip"] + _COMMON,
}


def short_name(name: str) -> str:
    """'void zg::prefill_kernel<4, false>(zg::PrefillParams)' -> 'prefill_kernel<4, false>'."""
    n = name.replace("(anonymous namespace)::", "")
    if n.startswith("void "):
        n = n[5:]
    n = n.split("(")[0]
    return n.replace("zg::", "")


def _ours(name: str) -> bool:
    return name.startswith("void zg::") or name.startswith("zg::")


def base_name(name: str) -> str:
    return short_name(name).split("<")[0]


def source_hash(kernel: str) -> str | None:
    files = KERNEL_SOURCES.get(base_name(kernel))
    if not files:
        return None
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(_CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def _per_dispatch_shape(csv_path: str, counter: str):
    """{(kernel name, grid size): [counter value per dispatch]}"""
    vals = defaultdict(list)
    with open(csv_path, newline="") as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                vals[(r["Kernel_Name"], int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
    return vals


def traffic(fetch_csv: str, write_csv: str, copy_bytes: int):
    """Mean HBM bytes per dispatch of each of our kernels (per grid size), scaled by the copy
    kernel's calibration."""
    fetch = _per_dispatch_shape(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch_shape(write_csv, "WRITE_SIZE")
    cf = [max(v) for k, v in fetch.items() if k[0].startswith(COPY_KERNEL)]
    cw = [max(v) for k, v in write.items() if k[0].startswith(COPY_KERNEL)]
    if not cf or not cw:
        raise SystemExit(f"no {COPY_KERNEL} dispatch in the counter files: cannot calibrate")
    f_scale = copy_bytes / (1024.0 * max(cf))   # the largest copy is the calibration copy
    w_scale = copy_bytes / (1024.0 * max(cw))
    out = []
    for k in sorted(set(fetch) & set(write)):
        if not _ours(k[0]):
            continue
        fb = sum(fetch[k]) / len(fetch[k]) * 1024.0 * f_scale
        wb = sum(write[k]) / len(write[k]) * 1024.0 * w_scale
        out.append({"kernel": short_name(k[0]), "grid": k[1], "fetch_bytes": round(fb),
                    "write_bytes": round(wb), "dispatches": len(fetch[k]),
                    "source_sha256": source_hash(k[0])})
    return out, f_scale, w_scale


def lookup_traffic(kernel: str, grid: int | None = None):
    """HBM bytes (fetch + write) per dispatch of `kernel` (at `grid` threads, if given) recorded
    in profiles/, or None when there is no unique record or the kernel's sources have changed
    since it was taken."""
    try:
        with open(TRAFFIC_JSON) as fh:
            recs = [r for r in json.load(fh)["kernels"] if r["kernel"] == kernel]
    except (OSError, KeyError, ValueError):
        return None
    if grid is not None:
        recs = [r for r in recs if r["grid"] == grid]
    if len(recs) != 1 or recs[0].get("source_sha256") != source_hash(kernel):
        return None
    return recs[0]["fetch_bytes"] + recs[0]["write_bytes"]


def _stats_md(trace_csv: str, cmd: str) -> str:
    """Per (kernel, grid size) dispatch statistics of our kernels and the device copy."""
    durs = defaultdict(list)
    with open(trace_csv, newline="") as fh:
        for r in csv.DictReader(fh):
            n = r["Kernel_Name"]
            if not (_ours(n) or n.startswith(COPY_KERNEL)):
                continue
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            durs[(short_name(n), grid)].append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    rows = sorted(durs.items(), key=lambda kv: -sum(kv[1]))
    lines = ["# rocprofv3 kernel-trace statistics", "", "Command:", "", "```", cmd, "```", "",
             "| kernel | grid (threads) | calls | avg (us) | min (us) | max (us) |",
             "|---|---:|---:|---:|---:|---:|"]
    for (n, g), d in rows:
        lines.append(f"| `{n}` | {g} | {len(d)} | {sum(d) / len(d):.1f} | {min(d):.1f} | "
                     f"{max(d):.1f} |")
    return "\n".join(lines) + "\n"


def _util_md(csv_paths, cmd: str) -> str:
    """Mean per-dispatch value of every counter in the given counter_collection files, for our
    kernels, plus per-wave instruction counts and wave-cycle fractions where the counters exist."""
    vals = defaultdict(lambda: defaultdict(list))
    for path in csv_paths:
        with open(path, newline="") as fh:
            for r in csv.DictReader(fh):
                if _ours(r["Kernel_Name"]):
                    key = (short_name(r["Kernel_Name"]), int(r["Grid_Size"]))
                    vals[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
    lines = ["# rocprofv3 SQ counters per dispatch", "", "Commands:", "", "```", cmd, "```", "",
             "Per-wave figures divide by SQ_WAVES; fractions of SQ_WAVE_CYCLES are per-wave time "
             "shares (waiting on s_waitcnt/barriers, waiting to issue, issuing).", ""]
    for (n, g), cs in sorted(vals.items()):
        m = {c: sum(v) / len(v) for c, v in cs.items()}
        lines += [f"## `{n}`, grid {g}", "", "| counter | mean per dispatch |", "|---|---:|"]
        lines += [f"| {c} | {v:.4g} |" for c, v in sorted(m.items())]
        waves = m.get("SQ_WAVES")
        if waves:
            for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_VALU_TRANS_F32"):
                if c in m:
                    lines.append(f"| {c} per wave | {m[c] / waves:.1f} |")
        wc = m.get("SQ_WAVE_CYCLES")
        if wc:
            for c in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU"):
                if c in m:
                    lines.append(f"| {c} / SQ_WAVE_CYCLES | {m[c] / wc:.3f} |")
        lines.append("")
    return "\n".join(lines) + "\n"


def main(argv):
    if "--" in argv:
        i = argv.index("--")
        argv, cmd = argv[:i], " ".join(argv[i + 1:])
    else:
        cmd = "(command not given)"
    if argv[0] == "stats":
        with open(argv[2], "w") as fh:
            fh.write(_stats_md(argv[1], cmd))
    elif argv[0] == "traffic":
        fetch_csv, write_csv, copy_bytes, out_json, out_md = argv[1:6]
        kern, fs, ws = traffic(fetch_csv, write_csv, int(copy_bytes))
        with open(out_json, "w") as fh:
            json.dump({"command": cmd, "copy_bytes": int(copy_bytes), "fetch_scale": fs,
                       "write_scale": ws, "kernels": kern}, fh, indent=1)
        lines = ["# HBM traffic per dispatch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
                 "Commands (two runs, one counter each):", "", "```", cmd, "```", "",
                 f"Calibration: for a device copy of {int(copy_bytes)} bytes in the same run the "
                 f"counters read 1/{fs:.4f} (FETCH_SIZE) and 1/{ws:.4f} (WRITE_SIZE) of its true "
                 "bytes; every figure below is the counter scaled by that factor.", "",
                 "| kernel | grid (threads) | dispatches | fetch (MB) | write (MB) | total (MB) |",
                 "|---|---:|---:|---:|---:|---:|"]
        for r in kern:
            lines.append(f"| `{r['kernel']}` | {r['grid']} | {r['dispatches']} | "
                         f"{r['fetch_bytes'] / 1e6:.1f} | {r['write_bytes'] / 1e6:.1f} | "
                         f"{(r['fetch_bytes'] + r['write_bytes']) / 1e6:.1f} |")
        with open(out_md, "w") as fh:
            fh.write("\n".join(lines) + "\n")
    elif argv[0] == "util":
        with open(argv[-1], "w") as fh:
            fh.write(_util_md(argv[1:-1], cmd))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
