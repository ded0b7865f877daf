"""Summaries of rocprofv3 CSV output (kernel statistics and HBM traffic counters).

  python -m mha_mla_kv_amd.profiling stats <kernel_stats.csv> --command "<cmd>"  > summary.md
  python -m mha_mla_kv_amd.profiling traffic <fetch_counter_collection.csv> <write_counter_collection.csv>
        --kernel <substring> --source-hash <hash> [--copy-bytes N] --command-fetch "<cmd>" --command-write "<cmd>"

FETCH_SIZE / WRITE_SIZE (KiB per dispatch) are scaled by what the same counter reads for a
plain device copy of known size (the `copy_1GiB` part of bench.py --copy-calibration, which
reads and writes `--copy-bytes` bytes): factor = bytes / (counter KiB * 1024).
"""
from __future__ import annotations

import argparse
import csv
import json
import statistics
import sys


def kernel_stats_md(path: str, command: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["# rocprofv3 kernel statistics", "", "Command:", "", "```", command, "```", "",
           "| kernel | calls | avg µs | min µs | max µs | % time |", "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        name = r["Name"].replace("attn::(anonymous namespace)::", "").replace("|", "/")
        if len(name) > 90:
            name = name[:87] + "..."
        out.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                   f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    return "\n".join(out) + "\n"


def _per_kernel(path: str, counter: str):
    vals = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return vals


def _pick(vals: dict, sub: str, largest: bool = False):
    keys = [k for k in vals if sub in k]
    if not keys:
        raise SystemExit(f"no dispatch of a kernel matching {sub!r}")
    if largest:
        keys.sort(key=lambda k: max(vals[k]))
        return vals[keys[-1]]
    if len(keys) > 1:
        raise SystemExit(f"kernel substring {sub!r} matches several kernels: {keys}")
    return vals[keys[0]]


def traffic(fetch_csv: str, write_csv: str, kernel: str, copy_bytes: int) -> dict:
    f, w = _per_kernel(fetch_csv, "FETCH_SIZE"), _per_kernel(write_csv, "WRITE_SIZE")
    # the copy calibration: the 1 GiB device copies, i.e. the copyBuffer dispatches within a
    # factor of two of the largest (the same kernel also serves the small input uploads)
    def big(vals):
        top = max(vals)
        return statistics.median([x for x in vals if x >= 0.5 * top])
    cf = big(_pick(f, "copyBuffer", largest=True))
    cw = big(_pick(w, "copyBuffer", largest=True))
    rf, rw = copy_bytes / (cf * 1024.0), copy_bytes / (cw * 1024.0)
    kf = statistics.median(_pick(f, kernel))
    kw = statistics.median(_pick(w, kernel))
    return {"fetch_kib_per_dispatch": kf, "write_kib_per_dispatch": kw,
            "copy_fetch_kib": cf, "copy_write_kib": cw, "fetch_factor": rf, "write_factor": rw,
            "read_bytes_per_launch": kf * 1024.0 * rf, "write_bytes_per_launch": kw * 1024.0 * rw,
            "bytes_per_launch": kf * 1024.0 * rf + kw * 1024.0 * rw}


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("--kernel", required=True, action="append")
    t.add_argument("--source-hash", required=True, action="append")
    t.add_argument("--copy-bytes", type=int, default=1 << 30)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        sys.stdout.write(kernel_stats_md(a.csv, a.command))
    else:
        res = {"_about": "HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE, each scaled by the "
                         "counter's reading for a plain 1 GiB device copy",
               "_commands": [a.command_fetch, a.command_write]}
        for k, h in zip(a.kernel, a.source_hash):
            e = traffic(a.fetch_csv, a.write_csv, k, a.copy_bytes)
            e["source_hash"] = h
            res[k] = e
        json.dump(res, sys.stdout, indent=1)
        sys.stdout.write("\n")


if __name__ == "__main__":
    main()
