"""Turn rocprofv3 output into the short summaries kept under ``profiles/``.

    python -m memory_efficient_long_amd.profiling stats RUN_kernel_stats.csv \
        --out profiles/NAME.md --cmd "the command that produced it"
    python -m memory_efficient_long_amd.profiling counters P1.csv P2.csv ... \
        --out profiles/NAME.md --kernels REGEX --cmd "the command"
    python -m memory_efficient_long_amd.profiling traffic --kernel attn_bwd_dkdv_kernel \
        --workload gpt1b-s128k --fetch F.csv --write W.csv --calib-fetch CF.csv \
        --calib-write CW.csv --copy-bytes N --out profiles/KERNEL_WORKLOAD_traffic.json

``traffic`` scales the FETCH_SIZE / WRITE_SIZE counters (KiB per dispatch) of
the kernel by what the same counters read for a device copy of a known number
of bytes (the calibration run of ``bench.py --calibrate-copy``), and records
the hash of the kernel sources so a later kernel change invalidates it.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import statistics
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(PKG_DIR, "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(name.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    name = re.sub(r"^void ", "", name)
    m = re.match(r"_ZN3bpt\d+(\w+?)I", name)
    base = m.group(1) if m else re.sub(r"[<(].*", "", name)
    return base


def cmd_stats(args) -> None:
    rows = list(csv.DictReader(open(args.csv)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = [f"# rocprofv3 kernel statistics: {args.title}", "",
             f"Command: `{args.cmd}`", "",
             "| kernel | calls | total ms | avg ms | % |", "|---|---|---|---|---|"]
    for r in rows[: args.top]:
        tot = float(r["TotalDurationNs"]) / 1e6
        lines.append(f"| `{r['Name'][:110]}` | {r['Calls']} | {tot:.3f} | "
                     f"{float(r['AverageNs']) / 1e6:.4f} | {100 * float(r['TotalDurationNs']) / total:.1f} |")
    lines += ["", f"Total kernel time: {total / 1e6:.3f} ms over all listed dispatches."]
    with open(args.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def _per_dispatch(path: str, counter: str, kernel_sub: str):
    vals = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        if kernel_sub not in r["Kernel_Name"]:
            continue
        key = r["Dispatch_Id"]
        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    return list(vals.values())


def cmd_traffic(args) -> None:
    fetch = _per_dispatch(args.fetch, "FETCH_SIZE", args.kernel)
    write = _per_dispatch(args.write, "WRITE_SIZE", args.kernel)
    cf = _per_dispatch(args.calib_fetch, "FETCH_SIZE", args.calib_kernel)
    cw = _per_dispatch(args.calib_write, "WRITE_SIZE", args.calib_kernel)
    if not (fetch and write and cf and cw):
        sys.exit("missing counter rows")
    kib_fetch_copy = statistics.median(cf)
    kib_write_copy = statistics.median(cw)
    f_scale = args.copy_bytes / kib_fetch_copy
    w_scale = args.copy_bytes / kib_write_copy
    rec = {
        "kernel": args.kernel, "workload": args.workload,
        "fetch_kib_per_dispatch": statistics.median(fetch),
        "write_kib_per_dispatch": statistics.median(write),
        "copy_bytes": args.copy_bytes,
        "copy_fetch_kib": kib_fetch_copy, "copy_write_kib": kib_write_copy,
        "fetch_scale_bytes_per_kib": f_scale, "write_scale_bytes_per_kib": w_scale,
        "hbm_bytes_per_launch": statistics.median(fetch) * f_scale + statistics.median(write) * w_scale,
        "kernel_source_hash": kernel_source_hash(),
        "command": args.cmd,
    }
    with open(args.out, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")


def cmd_counters(args) -> None:
    """Per-kernel medians (over dispatches) of the counters in one or more
    rocprofv3 --pmc runs, with a few ratios whose definitions are printed."""
    per = {}  # kernel -> counter -> {dispatch: value}
    for path in args.csv:
        for r in csv.DictReader(open(path)):
            if not re.search(args.kernels, r["Kernel_Name"]):
                continue
            name = args.aggregate or short_name(r["Kernel_Name"])
            d = per.setdefault(name, {}).setdefault(r["Counter_Name"], {})
            d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    names = sorted({c for k in per.values() for c in k})
    reduce = (lambda v: sum(v)) if args.aggregate else statistics.median
    med = {k: {c: reduce(list(v.values())) for c, v in cs.items()} for k, cs in per.items()}
    how = (f"Totals over all {max(len(v) for cs in per.values() for v in cs.values())} matching "
           "dispatches of one step." if args.aggregate else
           "Medians over the dispatches of each kernel (counter totals per dispatch).")
    lines = [f"# rocprofv3 counters: {args.title}", "", f"Command: `{args.cmd}`", "",
             how, "",
             "| counter | " + " | ".join(f"`{k}`" for k in med) + " |",
             "|---|" + "---|" * len(med)]
    for c in names:
        lines.append(f"| {c} | " + " | ".join(f"{med[k].get(c, float('nan')):.4g}" for k in med) + " |")
    ratios = [
        ("waiting share of wave cycles", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES"),
        ("LDS bank-conflict cycles per LDS-active cycle", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS"),
        ("VALU instructions per MFMA instruction", "SQ_INSTS_VALU", "SQ_INSTS_MFMA"),
        ("LDS instructions per MFMA instruction", "SQ_INSTS_LDS", "SQ_INSTS_MFMA"),
        ("L2 hit rate", "TCC_HIT_sum", ("TCC_HIT_sum", "TCC_MISS_sum")),
    ]
    lines += ["", "| ratio | " + " | ".join(f"`{k}`" for k in med) + " |",
              "|---|" + "---|" * len(med)]
    for label, num, den in ratios:
        vals = []
        for k in med:
            m = med[k]
            dv = sum(m.get(x, float("nan")) for x in den) if isinstance(den, tuple) else m.get(den, float("nan"))
            vals.append(f"{m.get(num, float('nan')) / dv:.3f}" if dv else "nan")
        lines.append(f"| {label} | " + " | ".join(vals) + " |")
    with open(args.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--out", required=True)
    s.add_argument("--cmd", default="")
    s.add_argument("--title", default="")
    s.add_argument("--top", type=int, default=25)
    t = sub.add_parser("traffic")
    for k in ("kernel", "workload", "fetch", "write", "calib_fetch", "calib_write", "out"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--calib-kernel", default="copy")
    t.add_argument("--cmd", default="")
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--out", required=True)
    c.add_argument("--kernels", default="attn_", help="regular expression on kernel names")
    c.add_argument("--aggregate", default="",
                   help="sum every matching dispatch into one column of this name")
    c.add_argument("--cmd", default="")
    c.add_argument("--title", default="")
    args = ap.parse_args()
    {"stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters}[args.cmd_name](args)


if __name__ == "__main__":
    main()
