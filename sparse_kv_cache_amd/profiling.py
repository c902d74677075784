"""Turns rocprofv3 CSV output into the short text summaries kept with the
repository, and computes the measured HBM traffic of the main scan kernel.

  python -m sparse_kv_cache_amd.profiling stats  <kernel_stats.csv> --command "..."
  python -m sparse_kv_cache_amd.profiling traffic --fetch <pmc.csv> --write <pmc.csv>
         --copy-mib M --budget B --out <file.json> --command "..."
  python -m sparse_kv_cache_amd.profiling counters <pmc.csv> [<pmc.csv> ...] --title T
         --command "..." [--command "..."]
  python -m sparse_kv_cache_amd.profiling trace <kernel_trace.csv> --last N --title T --command "..."

Traffic: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are read for the main
scan kernel and for a plain elementwise kernel that reads and writes exactly
M MiB.  Each counter is scaled by (known bytes / counter reading) of that copy,
so the figure is in real HBM bytes whatever unit or channel subset the
counter covers.  The result is tied to a digest of the kernel's source so a
stale figure is never reported for a changed kernel.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MAIN_KERNEL_SOURCES = ("scan.hip", "fathom_internal.h")


def source_digest() -> str:
    """Digest of the sources the main scan kernel is compiled from."""
    h = hashlib.sha256()
    for f in MAIN_KERNEL_SOURCES:
        with open(os.path.join(ROOT, "sparse_kv_cache_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    name = name.replace("fathom::(anonymous namespace)::", "")
    return name.split("(")[0].replace("void ", "")


def stats_markdown(path: str, command: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["# rocprofv3 kernel statistics", "", f"Source digest of the scan kernels: `{source_digest()}`", "",
           "Command:", "", "```", command, "```", "",
           "| kernel | calls | avg us | min us | max us | share % |",
           "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        out.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                   f"{float(r['Percentage']):.1f} |")
    return "\n".join(out) + "\n"


def _counter_rows(path: str, counter: str):
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            yield r["Kernel_Name"], float(r["Counter_Value"])


def _mean_for(path: str, counter: str, pattern: str, min_value: float = 0.0) -> float:
    vals = [v for name, v in _counter_rows(path, counter) if pattern in name and v >= min_value]
    if not vals:
        raise SystemExit(f"no {counter} rows for kernels matching {pattern!r} in {path}")
    return sum(vals) / len(vals)


def traffic(fetch_csv: str, write_csv: str, copy_mib: int, budget: int) -> dict:
    known_kib = copy_mib * 1024.0
    # the copy kernel's rows; the fill that creates its source writes only
    copy_fetch = _mean_for(fetch_csv, "FETCH_SIZE", "elementwise", known_kib / 4)
    copy_write = _mean_for(write_csv, "WRITE_SIZE", "elementwise", known_kib / 4)
    f_fetch, f_write = known_kib / copy_fetch, known_kib / copy_write
    main_fetch = _mean_for(fetch_csv, "FETCH_SIZE", "scan_main")
    main_write = _mean_for(write_csv, "WRITE_SIZE", "scan_main")
    read_b = main_fetch * f_fetch * 1024.0
    write_b = main_write * f_write * 1024.0
    return {
        "kernel": "scan_main_kernel",
        "budget": budget,
        "source_digest": source_digest(),
        "fetch_kib_per_dispatch": round(main_fetch, 3),
        "write_kib_per_dispatch": round(main_write, 3),
        "copy_mib": copy_mib,
        "copy_fetch_kib": round(copy_fetch, 3),
        "copy_write_kib": round(copy_write, 3),
        "fetch_scale": round(f_fetch, 5),
        "write_scale": round(f_write, 5),
        "read_bytes_per_launch": int(read_b),
        "write_bytes_per_launch": int(write_b),
        "bytes_per_launch": int(read_b + write_b),
    }


# rocprofv3's own definitions of the derived metrics reported (its counter
# list prints them); the other rows are raw SQ counters, summed over the
# GPU for one dispatch.
DERIVED = {
    "VALUBusy": "100*SQ_ACTIVE_INST_VALU/CU_NUM/GRBM_GUI_ACTIVE",
    "VALUUtilization": "100*SQ_THREAD_CYCLES_VALU/(SQ_ACTIVE_INST_VALU*MAX_WAVE_SIZE)",
    "LDSBankConflict": "100*SQ_LDS_BANK_CONFLICT/GRBM_GUI_ACTIVE/CU_NUM",
}


def counters_markdown(paths, title: str, commands) -> str:
    """Per-kernel mean of every counter in the pmc CSVs (one row per
    dispatch), plus ratios computed here with their formulas."""
    vals = {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            name = _short(r["Kernel_Name"])
            if not name.startswith("scan_"):
                continue
            vals.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    out = [f"# {title}", "", f"Source digest of the scan kernels: `{source_digest()}`", "", "Commands:", ""]
    for c in commands:
        out += ["```", c, "```", ""]
    for kernel in sorted(vals):
        cs = vals[kernel]
        mean = {c: sum(v) / len(v) for c, v in cs.items()}
        out += [f"## {kernel}", "", "| counter | mean per dispatch | dispatches |", "|---|---:|---:|"]
        for c in sorted(mean):
            out.append(f"| {c} | {mean[c]:.6g} | {len(cs[c])} |")
        derived = []
        if "SQ_INSTS_VALU" in mean and mean.get("SQ_INSTS_MFMA"):
            derived.append(("VALU instructions per MFMA", "SQ_INSTS_VALU / SQ_INSTS_MFMA",
                            mean["SQ_INSTS_VALU"] / mean["SQ_INSTS_MFMA"]))
        if "SQ_VALU_MFMA_BUSY_CYCLES" in mean and mean.get("SQ_BUSY_CU_CYCLES"):
            derived.append(("MFMA busy share of CU-busy cycles", "SQ_VALU_MFMA_BUSY_CYCLES / SQ_BUSY_CU_CYCLES",
                            mean["SQ_VALU_MFMA_BUSY_CYCLES"] / mean["SQ_BUSY_CU_CYCLES"]))
        if "SQ_LDS_BANK_CONFLICT" in mean and mean.get("SQ_INSTS_LDS"):
            derived.append(("bank-conflict cycles per LDS instruction", "SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS",
                            mean["SQ_LDS_BANK_CONFLICT"] / mean["SQ_INSTS_LDS"]))
        if "SQ_LDS_BANK_CONFLICT" in mean and mean.get("SQ_LDS_IDX_ACTIVE"):
            derived.append(("bank-conflict share of LDS-active cycles", "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE",
                            mean["SQ_LDS_BANK_CONFLICT"] / mean["SQ_LDS_IDX_ACTIVE"]))
        if "SQ_WAIT_INST_ANY" in mean and mean.get("SQ_WAVE_CYCLES"):
            derived.append(("waiting share of wave cycles", "SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES",
                            mean["SQ_WAIT_INST_ANY"] / mean["SQ_WAVE_CYCLES"]))
        if derived:
            out += ["", "| ratio | formula | value |", "|---|---|---:|"]
            out += [f"| {a} | `{b}` | {v:.4g} |" for a, b, v in derived]
        present = [k for k in DERIVED if k in mean]
        if present:
            out += ["", "Derived metrics above are rocprofv3's: " +
                    "; ".join(f"{k} = `{DERIVED[k]}`" for k in present) + "."]
        out.append("")
    return "\n".join(out) + "\n"


def trace_markdown(path: str, last: int, title: str, command: str) -> str:
    """Mean, min and max duration of the last `last` dispatches of each
    kernel in a kernel-trace CSV (the calls of the run's final phase)."""
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    by = {}
    for r in rows:
        by.setdefault(_short(r["Kernel_Name"]), []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = [f"# {title}", "", f"Source digest of the scan kernels: `{source_digest()}`", "", "Command:", "", "```",
           command, "```", "", f"Last {last} dispatches of each kernel (kernel trace):", "",
           "| kernel | dispatches | mean us | min us | max us |", "|---|---:|---:|---:|---:|"]
    for name in sorted(by, key=lambda n: -sum(by[n][-last:])):
        d = by[name][-last:]
        out.append(f"| {name} | {len(d)} | {sum(d) / len(d):.1f} | {min(d):.1f} | {max(d):.1f} |")
    return "\n".join(out) + "\n"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--budget", type=int, required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--command", action="append", default=[])
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--title", required=True)
    c.add_argument("--command", action="append", default=[])
    tr = sub.add_parser("trace")
    tr.add_argument("csv")
    tr.add_argument("--last", type=int, required=True)
    tr.add_argument("--title", required=True)
    tr.add_argument("--command", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        sys.stdout.write(trace_markdown(a.csv, a.last, a.title, a.command))
    elif a.cmd == "counters":
        sys.stdout.write(counters_markdown(a.csv, a.title, a.command))
    elif a.cmd == "stats":
        sys.stdout.write(stats_markdown(a.csv, a.command))
    else:
        rec = traffic(a.fetch, a.write, a.copy_mib, a.budget)
        rec["commands"] = a.command
        with open(a.out, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec))
    return 0


if __name__ == "__main__":
    sys.exit(main())
