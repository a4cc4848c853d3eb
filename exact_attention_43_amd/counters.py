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

MFMA, VALU and LDS activity per kernel against the clock actually run (one pass of
the counters listed in ``cmd_busy``)::

    python -m exact_attention_43_amd.counters busy DIR --kernel REGEX --out FILE.txt --cmd "..."
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


def cmd_busy(a):
    """Per kernel matching a.kernel (one line each): medians over its dispatches of the
    duration, the GPU clock actually run (GRBM_GUI_ACTIVE cycles / duration), the MFMA busy
    fraction against those cycles, the executed MFMA FLOPs (bf16 and FP8 MOPs x 512), the
    VALU-active cycles per SIMD and the LDS-active fraction per CU, from one counter pass:
    --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F8
    SQ_ACTIVE_INST_VALU SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE."""
    rx = re.compile(a.kernel)
    per = {}
    for r in _csvs(a.dir, "counter_collection.csv"):
        if not rx.search(r["Kernel_Name"]):
            continue
        d = per.setdefault((r["Kernel_Name"], r["Dispatch_Id"]), {})
        c, v = r["Counter_Name"], float(r["Counter_Value"])
        d[c] = d.get(c, 0.0) + v
        d["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    kernels = sorted({k[0] for k in per})
    if not kernels:
        raise SystemExit(f"no kernel matching {a.kernel!r}")
    med = lambda xs: statistics.median(xs)
    lines = [f"# MFMA, VALU and LDS activity per dispatch (medians); clock from GRBM_GUI_ACTIVE",
             f"# command: {a.cmd}", "",
             f"{'kernel':<64} {'disp':>4} {'us':>8} {'GHz':>5} {'mfma%':>6} {'TFLOP':>8} {'valu%':>6} "
             f"{'lds%':>5} {'bank%':>5}"]
    for k in kernels:
        ds = [v for (n, _), v in per.items() if n == k]
        ns = med([d["ns"] for d in ds])
        # GRBM_GUI_ACTIVE comes summed over the XCDs, which all count the same
        # cycles; over a short dispatch it also counts the collection window
        cyc = med([d["GRBM_GUI_ACTIVE"] for d in ds]) / a.xcds
        ghz = cyc / ns
        mfma = med([d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in ds]) / a.simds / cyc
        fl = med([(d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + d.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0)) * 512
                  for d in ds])
        valu = med([d["SQ_ACTIVE_INST_VALU"] for d in ds]) / a.simds / cyc
        lds = med([d["SQ_LDS_IDX_ACTIVE"] for d in ds]) / a.cus / cyc
        bank = med([d["SQ_LDS_BANK_CONFLICT"] for d in ds]) / max(1.0, med([d["SQ_LDS_IDX_ACTIVE"] for d in ds]))
        lines.append(f"{k[:64]:<64} {len(ds):>4} {ns / 1e3:>8.2f} {ghz:>5.2f} {100 * mfma:>6.1f} {fl / 1e12:>8.4f} "
                     f"{100 * valu:>6.1f} {100 * lds:>5.1f} {100 * bank:>5.1f}")
    lines += ["", "mfma%: SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE); valu%: SQ_ACTIVE_INST_VALU",
              "per SIMD over the same cycles (it counts every wave's VALU cycles, so two waves can exceed 100);",
              "lds%: SQ_LDS_IDX_ACTIVE per CU; bank%: SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE.",
              "GRBM_GUI_ACTIVE / 8 XCDs gives the cycles; over dispatches of a few tens of microseconds it also",
              "counts the collection window (the GHz column then reads high and the fractions low).",
              "Durations run longer under counter collection than in a plain run."]
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
    u = sub.add_parser("busy")
    u.add_argument("dir")
    u.add_argument("--kernel", required=True)
    u.add_argument("--simds", type=int, default=1024)
    u.add_argument("--cus", type=int, default=256)
    u.add_argument("--xcds", type=int, default=8)
    u.add_argument("--out", required=True)
    u.add_argument("--cmd", required=True)
    u.set_defaults(fn=cmd_busy)
    a = ap.parse_args(argv)
    a.fn(a)


if __name__ == "__main__":
    main(sys.argv[1:])
