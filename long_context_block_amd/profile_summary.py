"""Summaries of rocprofv3 CSV output for the library's kernels.

Reads the files rocprofv3 writes with ``--output-format csv`` (``*_kernel_stats.csv`` from a
``--kernel-trace --stats`` run, ``*_counter_collection.csv`` from ``--pmc`` runs) and writes

* a Markdown table of per-kernel launch statistics (``--stats``), and
* HBM traffic per launch from a FETCH_SIZE run and a WRITE_SIZE run, each scaled by what the same
  counter reads for a plain device copy of known size (``bench.py --copy-calibration BYTES``), as
  Markdown plus a JSON file that ``bench.py`` reads. The JSON records a digest of the kernel sources;
  ``bench.py`` ignores it once the sources have changed.
* SQ and texture counters per launch from two ``--pmc`` passes (instruction counts, VALU, MFMA and
  texture-address busy fractions, LDS bank conflicts), as Markdown.

Usage (from the repository root, on the host, after the GPU runs)::

    python -m long_context_block_amd.profile_summary stats DIR --title T --command C --out profiles/x.md
    python -m long_context_block_amd.profile_summary traffic --fetch DIR --write DIR --copy-fetch DIR \\
        --copy-write DIR --copy-bytes N --title T --command C --out-md profiles/y.md --out-json profiles/y.json
    python -m long_context_block_amd.profile_summary counters --pass-a DIR --pass-b DIR --title T \\
        --command C --out profiles/z.md
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# bench.py stage name -> kernel name fragments (the stage's launches)
STAGE_KERNELS = {
    "pyramid": ["pool_subtree_kernel", "pool_upper_kernel"],
    "route_planes": ["head_max_kernel", "split_f16_kernel"],
    "route_fused_leaf": [],  # route_kernel<..., true, ...>: the q_tile 1 walk with its own leaf stage
    "route": ["route_group_kernel", "route_lds_kernel", "route_kernel"],
    "regroup": ["hist_kernel", "scan_kernel", "scatter_kernel", "fill_zero_kernel"],
    "leaf_lse": ["leaf_lse_wg_kernel", "leaf_lse_kernel"],
    "finalize": ["finalize_kernel", "finalize_half_kernel"],
    "attn_leaf": ["attn_leaf_wg_kernel", "attn_leaf_kernel"],
    "attn_merge": ["attn_merge_kernel"],
    "bsa_select": ["bsa_kernel"],
    "decode_step": ["decode_kernel"],
    "attn_backward": ["bwd_prep_kernel", "attn_bwd_dq_kernel", "attn_bwd_dkdv_kernel", "bwd_dq_merge_kernel",
                      "bwd_finish_kernel"],
    "flat_leaf_lse": ["flat_leaf_lse_kernel"],
    "selection_quality": ["quality_kernel"],
    "pyramid_pooled": ["pool_leaf_kernel", "pool_level_kernel"],
    "select_variant": ["variant_walk_kernel"],
}


def source_digest(root: str = ROOT) -> str:
    """SHA-256 over the kernel sources and the ABI header (sorted paths and contents)."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(root, "long_context_block_amd", "csrc", "*")) +
                   glob.glob(os.path.join(root, "include", "*.h")))
    for f in files:
        h.update(os.path.relpath(f, root).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    name = name.strip('"')
    m = re.search(r"pisa::(\w+)(<[^(]*>)?", name)
    if m:
        return m.group(1) + (m.group(2) or "")
    return name.split("(")[0].replace("void ", "")[:60]


def stage_of(name: str) -> str | None:
    if re.search(r"\broute_kernel<[^>]*\btrue\b", name):
        return "route_fused_leaf"
    for stage, frags in STAGE_KERNELS.items():
        for f in frags:
            if re.search(r"\b" + f + r"\b", name):
                return stage
    return None


def _one(pattern: str) -> str:
    files = glob.glob(pattern, recursive=True)
    if not files:
        raise SystemExit(f"no file matches {pattern}")
    return sorted(files)[0]


def kernel_stats(d: str) -> list[dict]:
    rows = []
    with open(_one(os.path.join(d, "**", "*kernel_stats.csv"))) as f:
        for r in csv.DictReader(f):
            rows.append({"name": short_name(r["Name"]), "calls": int(r["Calls"]),
                         "avg_us": float(r["AverageNs"]) / 1e3, "total_us": float(r["TotalDurationNs"]) / 1e3,
                         "pct": float(r["Percentage"])})
    rows.sort(key=lambda x: -x["total_us"])
    return rows


def counter_per_launch(d: str, counter: str) -> dict[str, float]:
    """Average over launches of the counter summed over its instances, per kernel short name."""
    per = defaultdict(lambda: defaultdict(float))
    with open(_one(os.path.join(d, "**", "*counter_collection.csv"))) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            per[short_name(r["Kernel_Name"])][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in per.items()}


def cmd_stats(a):
    rows = kernel_stats(a.dir)
    if a.filter:
        rows = [r for r in rows if re.search(a.filter, r["name"])]
    lines = [f"# Kernel statistics: {a.title}", "", "Command (run from the repository root on one MI355X):", "",
             "```", a.command, "```", ""]
    if a.note:
        lines += [a.note, ""]
    lines += ["| Kernel | Calls | Average (us) | Total (us) | Share % |", "|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{r['name']}` | {r['calls']} | {r['avg_us']:.1f} | {r['total_us']:.1f} | {r['pct']:.2f} |")
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {a.out}")


def cmd_traffic(a):
    fetch = counter_per_launch(a.fetch, "FETCH_SIZE")
    write = counter_per_launch(a.write, "WRITE_SIZE")
    cf = counter_per_launch(a.copy_fetch, "FETCH_SIZE")
    cw = counter_per_launch(a.copy_write, "WRITE_SIZE")
    copy = [k for k in cf if "copyBuffer" in k or "copy" in k.lower()]
    if not copy:
        raise SystemExit("no copy kernel in the calibration runs")
    ck = copy[0]
    kib = a.copy_bytes / 1024.0
    f_fac, w_fac = kib / cf[ck], kib / cw[ck]
    kernels = {}
    for k in sorted(set(fetch) | set(write)):
        st = stage_of(k)
        if st is None:
            continue
        fb = fetch.get(k, 0.0) * f_fac * 1024.0
        wb = write.get(k, 0.0) * w_fac * 1024.0
        e = kernels.setdefault(st, {"kernels": [], "fetch_bytes": 0.0, "write_bytes": 0.0})
        e["kernels"].append(k)
        e["fetch_bytes"] += fb
        e["write_bytes"] += wb
    for e in kernels.values():
        e["bytes"] = e["fetch_bytes"] + e["write_bytes"]
    out = {"source_digest": source_digest(), "copy_kernel": ck, "copy_bytes": a.copy_bytes,
           "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4), "workload": a.workload,
           "command": a.command, "stages": kernels}
    with open(a.out_json, "w") as f:
        json.dump(out, f, indent=1)
    lines = [f"# HBM traffic per launch: {a.title}", "", "Commands (run from the repository root on one MI355X):",
             "", "```", a.command, "```", "",
             f"Calibration: a plain device copy of {a.copy_bytes} bytes (`{ck}`) reads FETCH_SIZE = "
             f"{cf[ck]:.0f} KiB and WRITE_SIZE = {cw[ck]:.0f} KiB per launch, so FETCH_SIZE is scaled by "
             f"{f_fac:.3f} and WRITE_SIZE by {w_fac:.3f}. Source digest of the measured build: "
             f"`{out['source_digest']}`.", "",
             "| Stage | Kernels | Read (GB) | Written (GB) | Total (GB) |", "|---|---|---|---|---|"]
    for st, e in sorted(kernels.items(), key=lambda kv: -kv[1]["bytes"]):
        lines.append(f"| {st} | {', '.join('`' + k + '`' for k in e['kernels'])} | {e['fetch_bytes'] / 1e9:.3f} | "
                     f"{e['write_bytes'] / 1e9:.3f} | {e['bytes'] / 1e9:.3f} |")
    with open(a.out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {a.out_md} and {a.out_json}")


# counters of the two passes (pass a: the SQ_WAVES row carries the launch's timestamps)
COUNTER_COLUMNS = ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
                   "SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_LDS_BANK_CONFLICT",
                   "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_LDS", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "TA_BUSY_avr",
                   "TD_TD_BUSY_avr"]


def counter_means(dirs: list[str]) -> tuple[dict, dict]:
    """Per kernel short name: the mean over its launches of every counter (summed over the counter's
    instances within a launch), and the mean launch duration in us (from the SQ_WAVES rows)."""
    per = defaultdict(lambda: defaultdict(lambda: defaultdict(float)))
    dur = defaultdict(dict)
    for d in dirs:
        with open(_one(os.path.join(d, "**", "*counter_collection.csv"))) as f:
            for r in csv.DictReader(f):
                k = short_name(r["Kernel_Name"])
                per[k][r["Counter_Name"]][(d, r["Dispatch_Id"])] += float(r["Counter_Value"])
                if r["Counter_Name"] == "SQ_WAVES":
                    dur[k][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    means = {k: {c: sum(v.values()) / len(v) for c, v in cs.items()} for k, cs in per.items()}
    durs = {k: sum(v.values()) / len(v) for k, v in dur.items() if v}
    return means, durs


def cmd_counters(a):
    means, durs = counter_means([a.pass_a, a.pass_b])
    lines = [f"# SQ and texture counters per launch: {a.title}", "",
             "Commands (run from the repository root on one MI355X; each pass is one bench step, and the "
             "launches of the step are averaged per kernel):", "", "```", a.command, "```", "",
             "Derived columns, read this way: *CU cycles* = SQ_BUSY_CU_CYCLES / 256 (cycles each CU was busy); "
             "*VALU busy* = 4 · SQ_ACTIVE_INST_VALU / (1024 SIMDs · CU cycles), with SQ_ACTIVE_INST_VALU counted "
             "in 4-cycle units (a wave64 VALU instruction issues over 4 cycles on a 16-lane SIMD; the counter "
             "tracks SQ_INSTS_VALU one to one); *MFMA busy* = SQ_VALU_MFMA_BUSY_CYCLES / (1024 · CU cycles); "
             "*TA busy* = TA_BUSY_avr / CU cycles; *LDS conflict* = SQ_LDS_BANK_CONFLICT / (256 · CU cycles). "
             "The fractions are relative to the cycles the CUs were busy, so for short launches with a ragged "
             "tail (finalize) they overstate the steady state. The launch time here is under the profiler and "
             "is slightly longer than in the timed bench.", "",
             "| Kernel | Launch (us) | VALU instr. (M) | of which MFMA (M) | transcendental (M) | VALU busy | "
             "MFMA busy | TA busy | LDS conflict |", "|---|---|---|---|---|---|---|---|---|"]
    order = sorted(means, key=lambda k: -durs.get(k, 0.0))
    for k in order:
        m = means[k]
        cu = m.get("SQ_BUSY_CU_CYCLES", 0.0) / 256
        if cu <= 0:
            continue
        g = lambda c: m.get(c, 0.0)
        lines.append(f"| `{k}` | {durs.get(k, 0.0):.0f} | {g('SQ_INSTS_VALU') / 1e6:.0f} | "
                     f"{g('SQ_INSTS_MFMA') / 1e6:.1f} | {g('SQ_INSTS_VALU_TRANS_F32') / 1e6:.1f} | "
                     f"{4 * g('SQ_ACTIVE_INST_VALU') / (1024 * cu):.0%} | "
                     f"{g('SQ_VALU_MFMA_BUSY_CYCLES') / (1024 * cu):.0%} | {g('TA_BUSY_avr') / cu:.0%} | "
                     f"{g('SQ_LDS_BANK_CONFLICT') / (256 * cu):.0%} |")
    cols = [c for c in COUNTER_COLUMNS if any(c in m for m in means.values())]
    lines += ["", "Raw averages per launch:", "", "| Kernel | " + " | ".join(cols) + " |",
              "|---|" + "---|" * len(cols)]
    for k in order:
        lines.append(f"| `{k}` | " + " | ".join(f"{means[k].get(c, 0.0):.4g}" for c in cols) + " |")
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {a.out}")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--note", default="")
    s.add_argument("--filter", default="", help="regex: keep only the kernels whose name matches")
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--workload", default="prefill_64k")
    t.add_argument("--title", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--out-md", required=True)
    t.add_argument("--out-json", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--pass-a", dest="pass_a", required=True)
    c.add_argument("--pass-b", dest="pass_b", required=True)
    c.add_argument("--title", required=True)
    c.add_argument("--command", required=True)
    c.add_argument("--out", required=True)
    a = ap.parse_args()
    {"stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters}[a.cmd](a)


if __name__ == "__main__":
    main()
