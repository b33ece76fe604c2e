"""Summaries of rocprofv3 output for the committed profiles.

Four subcommands, each reading the CSV files rocprofv3 writes with
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

  mfma    <pmc_dir> <trace_dir> <out.md> --command CMD
      Matrix-core use of the Newton-Schulz GEMMs on the GPT-2-124M hidden set
      from one pass with SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16,
      SQ_BUSY_CYCLES and GRBM_GUI_ACTIVE, with the kernel durations of a
      separate trace run beside it.

  chain   <dir> <out.md> --group LABEL:SKIP:COUNT ... --command CMD
      GPU-side anatomy of whole steps from <dir>/run_kernel_trace.csv: the
      trace is cut into steps (a momentum launch up to the next apply launch,
      in dispatch order); each group skips SKIP steps and summarises the next
      COUNT: the step's span on the GPU (momentum start to apply end), the
      time its kernels run, the idle time between them, the period from one
      step's start to the next, and the mean duration of each kernel family.

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
    (r"gram_reduce_kernel", "ns_gram_reduce"),
    (r"poly_update_kernel", "ns_poly_update"),
    (r"momentum_kernel", "momentum"),
    (r"norm_finalize_kernel", "norm_finalize"),
    (r"cast_kernel", "cast"),
    (r"apply_kernel", "apply"),
    (r"adamw_kernel", "adamw"),
    (r"untie_transpose_kernel", "untie"),
    (r"copyBuffer", "copy"),
    (r"ptr_patch_kernel", "ptr_patch"),
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
        fam, first, count, *label = w.split(":", 3)
        label = label[0] if label else "the benchmark's timed region"
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
        lines += ["", f"{fam} launches {first + 1}-{first + count} (in dispatch order; {label}): "
                      f"mean {mean:.2f} us, median {median:.2f} us over {count} launches."]
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


def read_dispatch_counters(d: str):
    """{dispatch_id: (kernel name, {counter: value})}; the CSV holds one value
    per dispatch and counter, summed over the counter's hardware instances."""
    out = {}
    with open(os.path.join(d, "run_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            key = int(r["Dispatch_Id"])
            name, vals = out.setdefault(key, (r["Kernel_Name"], collections.defaultdict(float)))
            vals[r["Counter_Name"]] += float(r["Counter_Value"])
    return out


def gpu_agent(d: str):
    with open(os.path.join(d, "run_agent_info.csv")) as f:
        for r in csv.DictReader(f):
            if r["Agent_Type"] == "GPU":
                return {"xcc": int(r["Num_Xcc"]), "simd": int(r["Simd_Count"]), "cu": int(r["Cu_Count"]),
                        "max_clk_mhz": float(r["Max_Engine_Clk_Fcompute"]), "target": r.get("Name", "")}
    raise SystemExit("no GPU agent in run_agent_info.csv")


def c3_ns_flops():
    """Algorithmic flops per launch of each Newton-Schulz GEMM on the
    GPT-2-124M hidden set (symmetry of X X^T and of A A counted once)."""
    from optimizer_muon_step_amd import workloads as wl
    gram = poly = upd = 0
    for s in wl.config_specs("c3"):
        m, n = min(s.rows, s.cols), max(s.rows, s.cols)
        gram += m * (m + 1) * n
        poly += m * m * (m + 1)
        upd += 2 * m * m * n
    return {"ns_gram": gram, "ns_poly": poly, "ns_update": upd}


def cmd_mfma(args):
    agent = gpu_agent(args.pmc_dir)
    disp = read_dispatch_counters(args.pmc_dir)
    trace = collections.defaultdict(list)
    for r in csv.DictReader(open(os.path.join(args.trace_dir, "run_kernel_trace.csv"))):
        trace[family(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    algo = c3_ns_flops()
    peak = 2.5e15
    lines = [f"# {args.title}", "", "Commands (from the repository root on an MI355X):", "", "```", args.command, "```", "",
             f"GPU: {agent['cu']} CUs, {agent['simd']} SIMDs, {agent['xcc']} XCDs, maximum engine clock "
             f"{agent['max_clk_mhz']:.0f} MHz.", "",
             "Normalisation.  SQ_VALU_MFMA_BUSY_CYCLES is summed over all SIMDs; GRBM_GUI_ACTIVE counts the "
             f"cycles the GPU was active in each of the {agent['xcc']} XCDs and the CSV holds their sum, so the "
             "kernel's active cycles are that sum / XCDs (rocprofv3's own MfmaUtil metric takes the per-XCD "
             "maximum).  MFMA utilisation = busy cycles / (active cycles x SIMDs): the fraction of the matrix "
             "pipes' cycles spent on MFMA work at the clock the kernel ran at.  Executed flops = "
             "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512.  The effective clock is active cycles / the kernel's mean "
             "duration in the trace run; utilisation x effective clock / 2.4 GHz x (algorithmic / executed "
             "flops) is the fraction of the 2.5 PFLOP/s bf16 peak the algorithmic flops reach, to be compared "
             "with algorithmic flops / trace duration / 2.5 PFLOP/s.", "",
             "| Kernel | Dispatches | Active cycles / dispatch | MFMA busy (SIMD-cycles) | MFMA utilisation | "
             "Executed GFLOP | Algorithmic GFLOP | Trace mean (us) | Effective clock (GHz) | "
             "Peak fraction from counters | Peak fraction from trace |",
             "|:--|--:|--:|--:|--:|--:|--:|--:|--:|--:|--:|"]
    for fam in ("ns_update", "ns_gram", "ns_poly"):
        rows = [v for n, v in disp.values() if family(n) == fam]
        if not rows:
            raise SystemExit(f"no {fam} dispatch in the counter run")
        k = len(rows)
        busy = sum(v["SQ_VALU_MFMA_BUSY_CYCLES"] for v in rows) / k
        mops = sum(v["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for v in rows) / k
        active = sum(v["GRBM_GUI_ACTIVE"] for v in rows) / k / agent["xcc"]
        util = busy / (active * agent["simd"])
        executed = 512.0 * mops
        durs = trace.get(fam)
        if not durs:
            raise SystemExit(f"no {fam} launch in the trace run")
        dur = sum(durs) / len(durs)
        clock = active / dur
        frac_counters = util * clock / 2.4e9 * algo[fam] / executed
        frac_trace = algo[fam] / dur / peak
        lines.append(f"| {fam} | {k} | {active:,.0f} | {busy:,.0f} | {100 * util:.1f}% | {executed / 1e9:.2f} | "
                     f"{algo[fam] / 1e9:.2f} | {dur * 1e6:.2f} | {clock / 1e9:.2f} | {frac_counters:.3f} | "
                     f"{frac_trace:.3f} |")
    lines += ["", f"Update-kernel fingerprint (sha256 of ns_gemm_tile.h, kernels_ns.hip and their build options): "
                  f"`{update_kernel_fingerprint()}`"]
    if args.note:
        lines += ["", args.note]
    open(args.out, "w").write("\n".join(lines) + "\n")


def cmd_chain(args):
    rows = list(csv.DictReader(open(os.path.join(args.dir, "run_kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    steps, cur = [], None
    for r in rows:
        fam = family(r["Kernel_Name"])
        if fam == "momentum":
            cur = []
        if cur is None:
            continue
        cur.append((fam, int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
        if fam == "apply":
            steps.append(cur)
            cur = None
    lines = [f"# {args.title}", "", "Command (from the repository root on an MI355X):", "", "```", args.command, "```", ""]
    if args.note:
        lines += [args.note, ""]
    lines += ["All times in microseconds, means over the steps of each group.  Span: first kernel start to last "
              "kernel end of a step.  Busy: sum of its kernels' durations.  Idle: span minus busy, the time "
              "between one kernel's end and the next one's start.  Period: one step's start to the next "
              "step's start (the last step of a group has none).", "",
              "| Workload | Steps | Launches per step | Span | Busy | Idle | Idle per launch | Period |",
              "|:--|--:|--:|--:|--:|--:|--:|--:|"]
    fam_tables = []
    pos = 0
    for g in args.group:
        label, skip, count = g.split(":")
        skip, count = int(skip), int(count)
        sel = steps[pos + skip:pos + skip + count]
        if len(sel) != count:
            raise SystemExit(f"group {g}: only {len(sel)} steps left in the trace")
        nxt = steps[pos + skip + 1:pos + skip + count + 1]
        pos += skip + count
        spans = [st[-1][2] - st[0][1] for st in sel]
        busy = [sum(e - b for _, b, e in st) for st in sel]
        periods = [n[0][1] - st[0][1] for st, n in zip(sel, nxt)][: count - 1]
        launches = sum(len(st) for st in sel) / count
        span, bsy = sum(spans) / count / 1e3, sum(busy) / count / 1e3
        idle = span - bsy
        period = sum(periods) / len(periods) / 1e3 if periods else float("nan")
        lines.append(f"| {label} | {count} | {launches:.1f} | {span:.1f} | {bsy:.1f} | {idle:.1f} | "
                     f"{idle / max(1.0, launches - 1):.2f} | {period:.1f} |")
        per = collections.defaultdict(list)
        for st in sel:
            for fam, b, e in st:
                per[fam].append((e - b) / 1e3)
        fam_tables.append((label, count, per))
    for label, count, per in fam_tables:
        lines += ["", f"{label}: kernel families per step", "", "| Family | Launches per step | Mean (us) | Per step (us) |",
                  "|:--|--:|--:|--:|"]
        for fam, d in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            lines.append(f"| {fam} | {len(d) / count:.1f} | {sum(d) / len(d):.2f} | {sum(d) / count:.1f} |")
    open(args.out, "w").write("\n".join(lines) + "\n")


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
                   help="FAMILY:FIRST:COUNT[:LABEL], mean duration of that family's launches FIRST..FIRST+COUNT-1")
    r = sub.add_parser("traffic")
    r.add_argument("fetch_dir")
    r.add_argument("write_dir")
    r.add_argument("out_json")
    r.add_argument("out_md")
    r.add_argument("--command", required=True)
    r.add_argument("--title", default="HBM traffic per dispatch")
    m = sub.add_parser("mfma")
    m.add_argument("pmc_dir")
    m.add_argument("trace_dir")
    m.add_argument("out")
    m.add_argument("--command", required=True)
    m.add_argument("--title", default="Matrix-core use of the Newton-Schulz GEMMs")
    m.add_argument("--note", default="")
    c = sub.add_parser("chain")
    c.add_argument("dir")
    c.add_argument("out")
    c.add_argument("--group", action="append", required=True, help="LABEL:SKIP:COUNT, in trace order")
    c.add_argument("--command", required=True)
    c.add_argument("--title", default="Step anatomy on the GPU")
    c.add_argument("--note", default="")
    args = ap.parse_args()
    {"trace": cmd_trace, "traffic": cmd_traffic, "mfma": cmd_mfma, "chain": cmd_chain}[args.cmd](args)


if __name__ == "__main__":
    main()
