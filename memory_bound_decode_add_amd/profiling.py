"""Summaries of rocprofv3 CSV output for the files kept under ``profiles/``.

    python -m memory_bound_decode_add_amd.profiling trace  TRACE_CSV --command CMD --out FILE.txt
    python -m memory_bound_decode_add_amd.profiling traffic --fetch CSV --write CSV \\
        --kernel SUBSTR --copy SUBSTR --copy-read-bytes R --copy-write-bytes W \\
        --bytes-per-launch B --command-fetch CMD --command-write CMD --out FILE.json

``trace`` reads a ``--kernel-trace`` CSV (``*_kernel_trace.csv``) and reports, per kernel
name and launch shape, the number of launches, the mean / median / min duration and the
median start-to-start interval between consecutive launches of that kernel (for
back-to-back launches, the quantity HIP events around a graph of them measure).

``traffic`` reads two ``--pmc`` CSVs (``*_counter_collection.csv``), one with FETCH_SIZE
and one with WRITE_SIZE (KiB per dispatch), averages them over the launches of the
kernel, and scales each by the ratio that makes a plain copy kernel of known size read
and write exactly its bytes.  The JSON it writes carries the hash of the kernel sources
it was taken on, so a later change to the kernel makes the figure stale.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
from collections import OrderedDict, defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEMV_SOURCES = ["memory_bound_decode_add_amd/csrc/w4_gemv.hip", "memory_bound_decode_add_amd/csrc/device_common.h"]


def source_hash(paths=GEMV_SOURCES) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _short(name: str, n: int = 90) -> str:
    return name if len(name) <= n else name[: n - 3] + "..."


def trace_summary(path: str):
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    groups: "OrderedDict[tuple, list]" = OrderedDict()
    prev_key, prev_start = None, None
    for r in rows:
        key = (r["Kernel_Name"], r.get("Workgroup_Size_X", r.get("Workgroup_Size", "")),
               r.get("Grid_Size_X", r.get("Grid_Size", "")))
        start, end = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        g = groups.setdefault(key, {"dur": [], "gap": []})
        g["dur"].append((end - start) / 1000.0)
        if key == prev_key:
            g["gap"].append((start - prev_start) / 1000.0)
        prev_key, prev_start = key, start
    out = []
    for (name, wg, grid), g in groups.items():
        d = g["dur"]
        out.append({"kernel": name, "workgroup": wg, "grid": grid, "launches": len(d),
                    "mean_us": statistics.mean(d), "median_us": statistics.median(d), "min_us": min(d),
                    "start_to_start_us": statistics.median(g["gap"]) if g["gap"] else None})
    out.sort(key=lambda e: -e["mean_us"] * e["launches"])
    return out


def write_trace_text(entries, command: str, out: str, top: int = 25):
    lines = ["rocprofv3 kernel trace summary", "", "command:", "  " + command, "",
             "per kernel and launch shape (durations in microseconds; start-to-start is the median",
             "interval between consecutive launches of the same kernel):", ""]
    for e in entries[:top]:
        s2s = f"{e['start_to_start_us']:.3f}" if e["start_to_start_us"] is not None else "-"
        lines.append(f"- {_short(e['kernel'])}")
        lines.append(f"    workgroup {e['workgroup']}, grid {e['grid']}: {e['launches']} launches, "
                     f"mean {e['mean_us']:.3f}, median {e['median_us']:.3f}, min {e['min_us']:.3f}, "
                     f"start-to-start {s2s}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def counter_means(path: str, counter: str):
    """Mean counter value per (kernel name, grid size): one kernel launched at several
    sizes gives several entries."""
    rows = list(csv.DictReader(open(path)))
    acc = defaultdict(list)
    for r in rows:
        if r["Counter_Name"] == counter:
            acc[(r["Kernel_Name"], int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
    return {k: statistics.mean(v) for k, v in acc.items()}


def _pick(means: dict, sub: str):
    hits = [(k, v) for k, v in means.items() if sub in k[0]]
    if len(hits) != 1:
        raise SystemExit(f"'{sub}' matches {len(hits)} kernel shapes: {[(k[0][:80], k[1]) for k, _ in hits]}")
    return hits[0]


def _pick_largest(means: dict, sub: str):
    """The largest-grid launch of the kernels matching sub: the calibration copy is the
    largest copy a profiled run makes (smaller copies of the same kernel may run too)."""
    hits = [(k, v) for k, v in means.items() if sub in k[0]]
    if not hits:
        raise SystemExit(f"'{sub}' matches no kernel")
    return max(hits, key=lambda kv: kv[0][1])


def traffic(a):
    fetch = counter_means(a.fetch, "FETCH_SIZE")
    write = counter_means(a.write, "WRITE_SIZE")
    (kf, _), f_k = _pick(fetch, a.kernel)
    _, w_k = _pick(write, a.kernel)
    _, f_c = _pick_largest(fetch, a.copy)
    _, w_c = _pick_largest(write, a.copy)
    ff = a.copy_read_bytes / (f_c * 1024.0)
    fw = a.copy_write_bytes / (w_c * 1024.0)
    hbm = f_k * 1024.0 * ff + w_k * 1024.0 * fw
    doc = {"kernel": kf, "kernel_source_hash": source_hash(),
           "fetch_kib_per_launch": f_k, "write_kib_per_launch": w_k,
           "copy_kernel": a.copy, "copy_fetch_kib": f_c, "copy_write_kib": w_c,
           "copy_read_bytes": a.copy_read_bytes, "copy_write_bytes": a.copy_write_bytes,
           "fetch_scale": ff, "write_scale": fw,
           "hbm_bytes_per_launch": hbm, "algorithmic_bytes_per_launch": a.bytes_per_launch,
           "traffic_over_algorithmic": hbm / a.bytes_per_launch if a.bytes_per_launch else None,
           "command_fetch": a.command_fetch, "command_write": a.command_write}
    with open(a.out, "w") as f:
        json.dump(doc, f, indent=1)
    print(json.dumps(doc, indent=1))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("csv")
    t.add_argument("--command", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--top", type=int, default=25)
    c = sub.add_parser("traffic")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--kernel", required=True)
    c.add_argument("--copy", required=True)
    c.add_argument("--copy-read-bytes", type=float, required=True)
    c.add_argument("--copy-write-bytes", type=float, required=True)
    c.add_argument("--bytes-per-launch", type=float, required=True)
    c.add_argument("--command-fetch", required=True)
    c.add_argument("--command-write", required=True)
    c.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.what == "trace":
        entries = trace_summary(a.csv)
        write_trace_text(entries, a.command, a.out, a.top)
        print(open(a.out).read())
    else:
        traffic(a)


if __name__ == "__main__":
    main()
