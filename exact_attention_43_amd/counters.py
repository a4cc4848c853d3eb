"""Summaries of rocprofv3 CSV output: kernel durations and HBM traffic per launch.

Kernel trace (``rocprofv3 --kernel-trace --stats -f csv``)::

    python -m exact_attention_43_amd.counters trace DIR --kernel REGEX --out FILE.txt --cmd "..."

HBM bytes per launch from two counter passes (``--pmc FETCH_SIZE`` then
``--pmc WRITE_SIZE``, both in KiB per dispatch), each scaled by what the same
counter reads for a plain device copy of known size (the copy leg of bench.py:
a 256 MiB fp32 multiply-by-one, which reads and writes 256 MiB each)::

    python -m exact_attention_43_amd.counters traffic --name NAME --kernel REGEX \\
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR --copy-bytes N \\
        --sources FILE ... --cmd "..." --out-dir profiles

writes ``NAME_traffic.json`` (read back by bench.py, and only trusted while the
sha256 of the listed kernel sources still matches) and ``NAME_traffic.txt``.

MFMA busy time and executed MFMA FLOPs from one counter pass
(``--pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16``)::

    python -m exact_attention_43_amd.counters mfma DIR --kernel REGEX --flops F --out FILE.txt --cmd "..."
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys


def _csvs(d, suffix):
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    rows = []
    for fn in files:
        with open(fn, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def kernel_stats(d, kernel_re):
    """Rows of the kernel statistics table whose name matches kernel_re."""
    rx = re.compile(kernel_re)
    out = []
    for r in _csvs(d, "kernel_stats.csv"):
        if rx.search(r["Name"]):
            out.append({"name": r["Name"], "calls": int(r["Calls"]),
                        "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                        "max_us": float(r["MaxNs"]) / 1e3, "total_us": float(r["TotalDurationNs"]) / 1e3})
    return out


def counter_values(d, counter, kernel_re):
    """Per-dispatch values of one counter for the kernels matching kernel_re, grouped by name."""
    rx = re.compile(kernel_re)
    per = {}
    for r in _csvs(d, "counter_collection.csv"):
        if r["Counter_Name"] != counter or not rx.search(r["Kernel_Name"]):
            continue
        key = (r["Kernel_Name"], r.get("Dispatch_Id", ""))
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])  # sum over dimensions
    groups = {}
    for (name, _), v in per.items():
        groups.setdefault(name, []).append(v)
    return groups


def _one_kernel(groups, what):
    if not groups:
        raise SystemExit(f"no dispatch found for {what}")
    if len(groups) > 1:
        names = ", ".join(f"{n[:60]}... ({len(v)})" for n, v in groups.items())
        raise SystemExit(f"{what}: several kernels match: {names}")
    (name, vals), = groups.items()
    return name, vals


def sha_of(paths, root):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(root, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def cmd_trace(a):
    rows = kernel_stats(a.dir, a.kernel)
    if not rows:
        raise SystemExit(f"no kernel matching {a.kernel!r}")
    lines = [f"# rocprofv3 kernel trace summary", f"# command: {a.cmd}", "",
             f"{'kernel':<72} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10}"]
    for r in rows:
        lines.append(f"{r['name'][:72]:<72} {r['calls']:>6} {r['avg_us']:>10.3f} {r['min_us']:>10.3f} "
                     f"{r['max_us']:>10.3f}")
    text = "\n".join(lines) + "\n"
    with open(a.out, "w") as f:
        f.write(text)
    print(text)


def cmd_traffic(a):
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    kname, fetch = _one_kernel(counter_values(a.fetch, "FETCH_SIZE", a.kernel), "FETCH_SIZE kernel")
    _, write = _one_kernel(counter_values(a.write, "WRITE_SIZE", a.kernel), "WRITE_SIZE kernel")
    cname, cfetch = _one_kernel(counter_values(a.copy_fetch, "FETCH_SIZE", a.copy_kernel),
                                "FETCH_SIZE copy")
    _, cwrite = _one_kernel(counter_values(a.copy_write, "WRITE_SIZE", a.copy_kernel), "WRITE_SIZE copy")
    kib = 1024.0
    f_fetch = a.copy_bytes / (statistics.median(cfetch) * kib)
    f_write = a.copy_bytes / (statistics.median(cwrite) * kib)
    fetch_b = statistics.median(fetch) * kib * f_fetch
    write_b = statistics.median(write) * kib * f_write
    rec = {
        "kernel": kname, "dispatches": [len(fetch), len(write)],
        "fetch_kib_median": statistics.median(fetch), "write_kib_median": statistics.median(write),
        "copy_kernel": cname, "copy_bytes": a.copy_bytes,
        "copy_fetch_kib_median": statistics.median(cfetch),
        "copy_write_kib_median": statistics.median(cwrite),
        "scale_fetch": round(f_fetch, 5), "scale_write": round(f_write, 5),
        "fetch_bytes_per_launch": round(fetch_b), "write_bytes_per_launch": round(write_b),
        "bytes_per_launch": round(fetch_b + write_b),
        "kernel_sha": sha_of(a.sources, root), "sources": a.sources, "command": a.cmd,
    }
    os.makedirs(a.out_dir, exist_ok=True)
    with open(os.path.join(a.out_dir, f"{a.name}_traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    text = (f"# HBM traffic per launch of {kname[:80]}\n# command: {a.cmd}\n\n"
            f"FETCH_SIZE median {rec['fetch_kib_median']:.1f} KiB over {len(fetch)} dispatches, "
            f"WRITE_SIZE median {rec['write_kib_median']:.1f} KiB over {len(write)} dispatches\n"
            f"copy calibration ({cname[:60]}, {a.copy_bytes} B each way): FETCH_SIZE "
            f"{rec['copy_fetch_kib_median']:.1f} KiB -> x{f_fetch:.4f}, WRITE_SIZE "
            f"{rec['copy_write_kib_median']:.1f} KiB -> x{f_write:.4f}\n"
            f"traffic per launch: read {fetch_b / 1e6:.3f} MB + write {write_b / 1e6:.3f} MB = "
            f"{(fetch_b + write_b) / 1e6:.3f} MB\n")
    with open(os.path.join(a.out_dir, f"{a.name}_traffic.txt"), "w") as f:
        f.write(text)
    print(text)


def cmd_mfma(a):
    """MFMA busy time per SIMD against the dispatch's duration, and MFMA FLOPs
    executed against the workload's algorithmic FLOPs, from one counter pass
    (SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16; one MOP is 512
    FLOPs).  The duration comes from the dispatch's own timestamps, which run
    longer under counter collection than in a plain run; the clock is the
    nominal peak clock, so the busy fraction is a lower bound."""
    rx = re.compile(a.kernel)
    per = {}
    for r in _csvs(a.dir, "counter_collection.csv"):
        if not rx.search(r["Kernel_Name"]):
            continue
        d = per.setdefault((r["Kernel_Name"], r["Dispatch_Id"]), {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        d["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    names = {k[0] for k in per}
    if len(names) != 1:
        raise SystemExit(f"expected one kernel for {a.kernel!r}, found {len(names)}")
    name = names.pop()
    disp = list(per.values())
    busy = statistics.median(d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in disp) / a.simds
    mops = statistics.median(d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for d in disp)
    ns = statistics.median(d["ns"] for d in disp)
    frac = busy / (ns * a.clock_ghz)
    lines = [
        f"# MFMA counters per dispatch of {name[:100]}",
        f"# command: {a.cmd}",
        "",
        f"dispatches: {len(disp)} (medians below)",
        f"SQ_VALU_MFMA_BUSY_CYCLES per SIMD: {busy:.0f} cycles ({a.simds} SIMDs)",
        f"dispatch duration under counter collection: {ns / 1e3:.2f} us",
        f"MFMA busy fraction at the nominal {a.clock_ghz} GHz: {100 * frac:.1f}%",
        f"MFMA FLOPs executed (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512): {mops * 512:.4g}",
    ]
    if a.flops:
        lines.append(f"algorithmic FLOPs: {a.flops:.4g}; executed / algorithmic = {mops * 512 / a.flops:.3f} "
                     "(masked blocks on the mask boundary are computed whole)")
    text = "\n".join(lines) + "\n"
    with open(a.out, "w") as f:
        f.write(text)
    print(text)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--kernel", default=".")
    t.add_argument("--out", required=True)
    t.add_argument("--cmd", required=True)
    t.set_defaults(fn=cmd_trace)
    r = sub.add_parser("traffic")
    r.add_argument("--name", required=True)
    r.add_argument("--kernel", required=True)
    r.add_argument("--fetch", required=True)
    r.add_argument("--write", required=True)
    r.add_argument("--copy-fetch", required=True)
    r.add_argument("--copy-write", required=True)
    r.add_argument("--copy-kernel", default="MulFunctor|mul")
    r.add_argument("--copy-bytes", type=int, default=256 << 20)
    r.add_argument("--sources", nargs="+", required=True)
    r.add_argument("--cmd", required=True)
    r.add_argument("--out-dir", default="profiles")
    r.set_defaults(fn=cmd_traffic)
    m = sub.add_parser("mfma")
    m.add_argument("dir")
    m.add_argument("--kernel", required=True)
    m.add_argument("--flops", type=float, default=0.0)
    m.add_argument("--simds", type=int, default=1024)
    m.add_argument("--clock-ghz", type=float, default=2.4)
    m.add_argument("--out", required=True)
    m.add_argument("--cmd", required=True)
    m.set_defaults(fn=cmd_mfma)
    a = ap.parse_args(argv)
    a.fn(a)


if __name__ == "__main__":
    main(sys.argv[1:])
