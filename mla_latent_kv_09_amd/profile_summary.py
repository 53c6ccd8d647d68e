"""Summarise rocprofv3 result databases (rocpd SQLite) as short markdown tables.

    python -m mla_latent_kv_09_amd.profile_summary trace DB [--regex R]
    python -m mla_latent_kv_09_amd.profile_summary counters DB [DB ...] [--regex R]
    python -m mla_latent_kv_09_amd.profile_summary traffic --fetch DB --write DB
            --calib-fetch DB --calib-write DB --calib-mib N --regex R
    python -m mla_latent_kv_09_amd.profile_summary clock DB [--regex R] [--flops-per-dispatch F]

`trace` lists per-kernel dispatch count and duration statistics from a
`--kernel-trace` run; `counters` lists per-kernel mean counter values per
dispatch from `--pmc` runs; `traffic` turns FETCH_SIZE / WRITE_SIZE (KiB per
dispatch) into HBM bytes per dispatch, each scaled by what the same counter
reads for a plain copy of known size; `clock` divides GRBM_GUI_ACTIVE (GPU
cycles of a dispatch) by the dispatch's duration, giving the clock the chip ran
at, and with SQ_VALU_MFMA_BUSY_CYCLES (summed over the 32 SIMDs of a shader
engine) the matrix pipes' busy fraction at that clock.
"""
from __future__ import annotations

import argparse
import collections
import glob
import hashlib
import json
import os
import re
import sqlite3
import statistics

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def _db(path: str) -> str:
    if os.path.isdir(path):
        found = glob.glob(os.path.join(path, "**", "*_results.db"), recursive=True)
        if not found:
            raise SystemExit(f"no *_results.db under {path}")
        return found[0]
    return path


def _short(name: str) -> str:
    name = re.sub(r"\(anonymous namespace\)::", "", name)
    return name if len(name) <= 70 else name[:67] + "..."


def kernel_durations(path: str, regex: str = "."):
    con = sqlite3.connect(_db(path))
    out = collections.defaultdict(list)
    for name, dur in con.execute("select name, duration from kernels"):
        if re.search(regex, name):
            out[name].append(dur / 1000.0)  # ns -> us
    return out


def counter_means(paths, regex: str = "."):
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in paths:
        con = sqlite3.connect(_db(path))
        for name, counter, value in con.execute(
                "select name, counter_name, counter_value from pmc_events"):
            if re.search(regex, name):
                out[name][counter].append(value)
    return {k: {c: statistics.fmean(v) for c, v in d.items()} for k, d in out.items()}


def cmd_trace(args):
    d = kernel_durations(args.db, args.regex)
    print("| kernel | dispatches | mean us | median us | min us | max us |")
    print("|---|---|---|---|---|---|")
    for name, v in sorted(d.items(), key=lambda kv: -sum(kv[1])):
        print(f"| `{_short(name)}` | {len(v)} | {statistics.fmean(v):.2f} | "
              f"{statistics.median(v):.2f} | {min(v):.2f} | {max(v):.2f} |")


def cmd_counters(args):
    d = counter_means(args.db, args.regex)
    counters = sorted({c for v in d.values() for c in v})
    print("| kernel | " + " | ".join(counters) + " |")
    print("|---|" + "---|" * len(counters))
    for name, v in sorted(d.items()):
        print(f"| `{_short(name)}` | " + " | ".join(f"{v.get(c, float('nan')):.1f}" for c in counters) + " |")


def dispatch_counters(path: str, regex: str = "."):
    """{kernel: [(duration ns, {counter: mean over instances})]} per dispatch."""
    con = sqlite3.connect(_db(path))
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    dur, names = {}, {}
    for name, did, d, counter, value in con.execute(
            "select name, dispatch_id, duration, counter_name, counter_value from pmc_events"):
        if re.search(regex, name):
            per[did][counter].append(value)
            dur[did], names[did] = d, name
    out = collections.defaultdict(list)
    for did, cs in per.items():
        out[names[did]].append((dur[did], {c: statistics.fmean(v) for c, v in cs.items()}))
    return out


def cmd_clock(args):
    d = dispatch_counters(args.db, args.regex)
    print("| kernel | dispatches | mean us | GRBM_GUI_ACTIVE | clock GHz | MFMA busy | TFLOP/s |")
    print("|---|---|---|---|---|---|---|")
    for name, rows in sorted(d.items(), key=lambda kv: -sum(r[0] for r in kv[1])):
        us = statistics.fmean(r[0] for r in rows) / 1000.0
        gui = statistics.fmean(r[1].get("GRBM_GUI_ACTIVE", float("nan")) for r in rows)
        ghz = statistics.fmean(r[1].get("GRBM_GUI_ACTIVE", float("nan")) / r[0] for r in rows)
        busy = statistics.fmean(r[1].get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / 32.0
                                / r[1].get("GRBM_GUI_ACTIVE", float("nan")) for r in rows)
        tf = args.flops_per_dispatch / (us * 1e-6) / 1e12 if args.flops_per_dispatch else float("nan")
        print(f"| `{_short(name)}` | {len(rows)} | {us:.2f} | {gui:.0f} | {ghz:.3f} | {busy:.3f} | {tf:.0f} |")


def cmd_traffic(args):
    mib_kib = args.calib_mib * 1024.0
    cf = counter_means([args.calib_fetch], args.calib_regex)
    cw = counter_means([args.calib_write], args.calib_regex)
    fetch_copy = max(v["FETCH_SIZE"] for v in cf.values() if "FETCH_SIZE" in v)
    write_copy = max(v["WRITE_SIZE"] for v in cw.values() if "WRITE_SIZE" in v)
    f_scale = mib_kib / fetch_copy
    w_scale = mib_kib / write_copy
    fk = counter_means([args.fetch], args.regex)
    wk = counter_means([args.write], args.regex)
    rows = {}
    for name in sorted(set(fk) | set(wk)):
        fetch = fk.get(name, {}).get("FETCH_SIZE", float("nan")) * f_scale * 1024
        write = wk.get(name, {}).get("WRITE_SIZE", float("nan")) * w_scale * 1024
        rows[name] = {"fetch_bytes": fetch, "write_bytes": write, "bytes_per_launch": fetch + write}
    print(json.dumps({"fetch_scale": f_scale, "write_scale": w_scale,
                      "copy_fetch_kib": fetch_copy, "copy_write_kib": write_copy,
                      "kernels": rows}, indent=1))
    if args.record:
        # One record per (kernel, workload): the named kernel's bytes per launch, tagged with
        # its source's hash so that a later source change invalidates it.
        match = [n for n in rows if re.search(args.record_regex, n)]
        if len(match) != 1:
            raise SystemExit(f"--record-regex matches {len(match)} kernels: {match}")
        r = rows[match[0]]
        with open(os.path.join(CSRC, args.kernel_source), "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()[:16]
        rec = {"workload": args.workload, "num_splits": args.num_splits, "kernel": args.kernel_name,
               "kernel_source_sha256_16": sha, "bytes_per_launch": r["bytes_per_launch"],
               "fetch_bytes": r["fetch_bytes"], "write_bytes": r["write_bytes"],
               "fetch_scale": f_scale, "write_scale": w_scale, "source": args.summary}
        try:
            with open(args.record) as f:
                data = json.load(f)
        except OSError:
            data = {"records": []}
        data["records"] = [x for x in data.get("records", [])
                           if not (x.get("kernel") == rec["kernel"] and x.get("workload") == rec["workload"])]
        data["records"].append(rec)
        with open(args.record, "w") as f:
            json.dump(data, f, indent=1)
            f.write("\n")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--regex", default=".")
    c = sub.add_parser("counters")
    c.add_argument("db", nargs="+")
    c.add_argument("--regex", default=".")
    k = sub.add_parser("clock")
    k.add_argument("db")
    k.add_argument("--regex", default=".")
    k.add_argument("--flops-per-dispatch", type=float, default=0.0)
    f = sub.add_parser("traffic")
    f.add_argument("--fetch", required=True)
    f.add_argument("--write", required=True)
    f.add_argument("--calib-fetch", required=True)
    f.add_argument("--calib-write", required=True)
    f.add_argument("--calib-mib", type=float, required=True)
    f.add_argument("--calib-regex", default="copyBuffer")
    f.add_argument("--regex", default=".")
    f.add_argument("--record", help="records file to update (e.g. profiles/traffic_decode.json)")
    f.add_argument("--record-regex", default="decode", help="the one kernel the record is for")
    f.add_argument("--kernel-name", default="decode_m32_kernel")
    f.add_argument("--kernel-source", default="decode_m32.hip", help="file under csrc/")
    f.add_argument("--workload", default="")
    f.add_argument("--num-splits", type=int, default=0)
    f.add_argument("--summary", default="", help="the profiles/ summary the record comes from")
    args = ap.parse_args()
    {"trace": cmd_trace, "counters": cmd_counters, "traffic": cmd_traffic, "clock": cmd_clock}[args.cmd](args)


if __name__ == "__main__":
    main()
