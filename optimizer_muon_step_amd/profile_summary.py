"""Summaries of rocprofv3 output for the committed profiles.

Two subcommands, each reading the CSV files rocprofv3 writes with
`--output-format csv -o run`:

  trace   <dir> <out.md> --command CMD
      Kernel table from <dir>/run_kernel_stats.csv (calls, mean/min/max ns).

  traffic <fetch_dir> <write_dir> <out.json> <out.md> --command CMD
      HBM-side bytes per dispatch of every kernel family from one FETCH_SIZE
      pass and one WRITE_SIZE pass.  Both counters are calibrated against the
      largest plain device copy in the same run (a 256 MiB buffer copied once by
      bench.py after its timed region): factor = known bytes / counted bytes.
      The JSON holds the figure bench.py reports as `roofline.traffic` for the
      update GEMM, tagged with the sha256 of the kernel source it was taken on.

FETCH_SIZE and WRITE_SIZE count traffic between the L2 caches and the memory
fabric, so reads served by the memory-side cache count as fetched.
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import re

from optimizer_muon_step_amd.build import update_kernel_fingerprint

HERE = os.path.dirname(os.path.abspath(__file__))
CALIB_BYTES = 64 * 1024 * 1024 * 4   # bench.py's calibration copy: 64M fp32

FAMILIES = [
    (r"ns_gemm_kernel<0\b", "ns_gram"),
    (r"ns_gemm_kernel<1\b", "ns_poly"),
    (r"ns_gemm_kernel<2\b", "ns_update"),
    (r"momentum_kernel", "momentum"),
    (r"norm_finalize_kernel", "norm_finalize"),
    (r"cast_kernel", "cast"),
    (r"apply_kernel", "apply"),
    (r"adamw_kernel", "adamw"),
    (r"untie_transpose_kernel", "untie"),
    (r"copyBuffer", "copy"),
]


def family(name: str) -> str:
    for pat, fam in FAMILIES:
        if re.search(pat, name):
            return fam
    return "other"


def read_counters(d: str, counter: str):
    """{dispatch_id: (kernel name, value)} for one counter."""
    out = {}
    with open(os.path.join(d, "run_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            key = int(r["Dispatch_Id"])
            name, val = r["Kernel_Name"], float(r["Counter_Value"])
            prev = out.get(key)
            out[key] = (name, val + (prev[1] if prev else 0.0))
    return out


def cmd_trace(args):
    rows = list(csv.DictReader(open(os.path.join(args.dir, "run_kernel_stats.csv"))))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = [f"# {args.title}", "", "Command (from the repository root on an MI355X):", "", "```", args.command, "```", ""]
    if args.note:
        lines += [args.note, ""]
    lines += ["| Kernel | Calls | Mean (us) | Min (us) | Max (us) | Share |", "|:--|--:|--:|--:|--:|--:|"]
    for r in rows:
        name = r["Name"].split("(")[0]
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{100 * float(r['TotalDurationNs']) / total:.1f}% |")
    for w in args.window or []:
        fam, first, count = w.split(":")
        first, count = int(first), int(count)
        trace = [r for r in csv.DictReader(open(os.path.join(args.dir, "run_kernel_trace.csv")))
                 if family(r["Kernel_Name"]) == fam]
        trace.sort(key=lambda r: int(r["Dispatch_Id"]))
        sel = trace[first:first + count]
        if len(sel) != count:
            raise SystemExit(f"window {w}: only {len(sel)} launches")
        durs = sorted((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in sel)
        mean = sum(durs) / count
        median = (durs[(count - 1) // 2] + durs[count // 2]) / 2
        lines += ["", f"{fam} launches {first + 1}-{first + count} (in dispatch order; the benchmark's timed "
                      f"region): mean {mean:.2f} us, median {median:.2f} us over {count} launches."]
    open(args.out, "w").write("\n".join(lines) + "\n")


def cmd_traffic(args):
    fetch = read_counters(args.fetch_dir, "FETCH_SIZE")
    write = read_counters(args.write_dir, "WRITE_SIZE")

    def calib(table):
        copies = [v for n, v in table.values() if family(n) == "copy"]
        if not copies:
            raise SystemExit("no copy dispatch found for calibration")
        return CALIB_BYTES / (max(copies) * 1024.0)

    f_fac, w_fac = calib(fetch), calib(write)
    fams = collections.defaultdict(lambda: {"n_fetch": 0, "fetch_kib": 0.0, "n_write": 0, "write_kib": 0.0})
    for n, v in fetch.values():
        e = fams[family(n)]
        e["n_fetch"] += 1
        e["fetch_kib"] += v
    for n, v in write.values():
        e = fams[family(n)]
        e["n_write"] += 1
        e["write_kib"] += v
    per = {}
    for fam, e in fams.items():
        fk = e["fetch_kib"] / max(1, e["n_fetch"])
        wk = e["write_kib"] / max(1, e["n_write"])
        per[fam] = {"dispatches": e["n_fetch"], "fetch_kib_raw": round(fk, 1), "write_kib_raw": round(wk, 1),
                    "fetch_bytes": round(fk * 1024 * f_fac), "write_bytes": round(wk * 1024 * w_fac)}
    upd = per.get("ns_update")
    if upd is None:
        raise SystemExit("no update-GEMM dispatch in the counter runs")
    sha = update_kernel_fingerprint()
    rec = {
        "kernel": "ns_update",
        "kernel_source_sha256": sha,
        "hbm_bytes_per_launch": upd["fetch_bytes"] + upd["write_bytes"],
        "fetch_bytes_per_launch": upd["fetch_bytes"],
        "write_bytes_per_launch": upd["write_bytes"],
        "calibration": {"copy_bytes_each_way": CALIB_BYTES, "fetch_factor": round(f_fac, 4),
                        "write_factor": round(w_fac, 4)},
        "families": per,
        "command": args.command,
    }
    json.dump(rec, open(args.out_json, "w"), indent=1)
    lines = [f"# {args.title}", "", "Commands (from the repository root on an MI355X):", "", "```", args.command, "```", "",
             f"Calibration: a plain device copy of {CALIB_BYTES >> 20} MiB in the same run reads "
             f"{CALIB_BYTES >> 20} MiB and writes {CALIB_BYTES >> 20} MiB; the counters gave "
             f"FETCH factor {f_fac:.3f} and WRITE factor {w_fac:.3f} (known bytes / counted bytes).", "",
             "| Kernel family | Dispatches | FETCH_SIZE raw (KiB) | WRITE_SIZE raw (KiB) | Read (MB, calibrated) | Written (MB, calibrated) |",
             "|:--|--:|--:|--:|--:|--:|"]
    for fam in sorted(per, key=lambda k: -(per[k]["fetch_bytes"] + per[k]["write_bytes"])):
        p = per[fam]
        lines.append(f"| {fam} | {p['dispatches']} | {p['fetch_kib_raw']:.0f} | {p['write_kib_raw']:.0f} | "
                     f"{p['fetch_bytes'] / 1e6:.1f} | {p['write_bytes'] / 1e6:.1f} |")
    lines += ["", f"Update-kernel fingerprint (sha256 of ns_gemm_tile.h, kernels_ns.hip and their build options): `{sha}`"]
    open(args.out_md, "w").write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("out")
    t.add_argument("--command", required=True)
    t.add_argument("--title", default="Kernel trace summary")
    t.add_argument("--note", default="")
    t.add_argument("--window", action="append",
                   help="FAMILY:FIRST:COUNT, mean duration of that family's launches FIRST..FIRST+COUNT-1")
    r = sub.add_parser("traffic")
    r.add_argument("fetch_dir")
    r.add_argument("write_dir")
    r.add_argument("out_json")
    r.add_argument("out_md")
    r.add_argument("--command", required=True)
    r.add_argument("--title", default="HBM traffic per dispatch")
    args = ap.parse_args()
    (cmd_trace if args.cmd == "trace" else cmd_traffic)(args)


if __name__ == "__main__":
    main()
