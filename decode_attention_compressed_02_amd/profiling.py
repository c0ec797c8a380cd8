"""Turn rocprofv3 CSV output into the short text summaries kept with the
benchmark: per-kernel duration statistics, and HBM traffic per launch of a
kernel from the FETCH_SIZE / WRITE_SIZE counters.

The counters report KiB per dispatch.  They are calibrated against a plain
device copy of known size run in the same process (``bench.py
--copy-calibration-mib``): the scale factor is (bytes the copy must move) /
(bytes the counter reports for it), separately for reads and writes.

Usage (after the rocprofv3 runs listed in the summary itself):
  python -m decode_attention_compressed_02_amd.profiling stats <kernel_stats.csv>
  python -m decode_attention_compressed_02_amd.profiling traffic \\
      --fetch <fetch counter_collection.csv> --write <write counter_collection.csv> \\
      --kernel k_split --copy-mib 512 --workload "..." --out profiles/split_kernel_traffic.json
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# sources that define the split kernel; a traffic figure is valid only for them
KERNEL_SOURCES = [os.path.join(ROOT, "decode_attention_compressed_02_amd", "csrc", f)
                  for f in ("split_kernel.h", "decode.hip", "swan_internal.h")
                  + tuple(f"split_g{g}{p}.hip" for g in (1, 2, 4, 8) for p in ("", "_paged"))]
COPY_KERNEL_HINT = "copy"  # torch's device-to-device copy kernel names contain this


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stats_table(path: str, top: int = 12) -> str:
    """Markdown table of a rocprofv3 kernel_stats.csv."""
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = ["| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows[:top]:
        out.append("| {} | {} | {:.2f} | {:.2f} | {:.2f} | {:.1f} |".format(
            r["Name"][:80].replace("|", "/"), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return "\n".join(out)


def last_dispatches(trace_csv: str, kernel: str, last: int, skip: int = 0):
    """(mean, min, max) duration in us of `last` dispatches of a kernel in a
    rocprofv3 kernel_trace.csv (in start order), ending `skip` dispatches
    before the run's last one."""
    rows = [r for r in csv.DictReader(open(trace_csv)) if kernel in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    rows = rows[:len(rows) - skip] if skip else rows
    d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows[-last:]]
    return statistics.mean(d), min(d), max(d), len(rows) + skip


def dispatch_series(trace_csv: str, kernel: str, first: int, per_bin: int):
    """Durations (us) of the first `first` dispatches of a kernel in a
    rocprofv3 kernel_trace.csv, in start order, as (first index, last index,
    mean, min, max) per bin of `per_bin` dispatches."""
    rows = [r for r in csv.DictReader(open(trace_csv)) if kernel in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows[:first]]
    out = []
    for i in range(0, len(d), per_bin):
        c = d[i:i + per_bin]
        out.append((i, i + len(c) - 1, statistics.mean(c), min(c), max(c)))
    return out, len(rows)


def clock_series(trace_csv: str, counter_csv: str, kernel: str, per_bin: int, xcds: int = 8):
    """Shader clock of each dispatch of a kernel, from a run that collected
    GRBM_GUI_ACTIVE (GPU-busy cycles, summed over the XCDs) together with the
    kernel trace: cycles per XCD / duration.  Returns (first index, last
    index, mean duration us, mean clock GHz) per bin of `per_bin` dispatches
    in start order."""
    cyc = {}
    for r in csv.DictReader(open(counter_csv)):
        if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
            cyc[int(r["Dispatch_Id"])] = float(r["Counter_Value"])
    rows = [r for r in csv.DictReader(open(trace_csv)) if kernel in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    pts = []
    for r in rows:
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        c = cyc.get(int(r["Dispatch_Id"]))
        if c:
            pts.append((dur, c / xcds / dur / 1e3))
    out = []
    for i in range(0, len(pts), per_bin):
        c = pts[i:i + per_bin]
        out.append((i, i + len(c) - 1, statistics.mean(x[0] for x in c), statistics.mean(x[1] for x in c)))
    return out


def counter_means(counter_csv: str, kernel: str, last: int) -> dict:
    """{counter: mean value per dispatch} over the last `last` dispatches of a
    kernel in a rocprofv3 counter_collection.csv."""
    per = {}
    for r in csv.DictReader(open(counter_csv)):
        if kernel in r["Kernel_Name"]:
            per.setdefault(int(r["Dispatch_Id"]), {})[r["Counter_Name"]] = float(r["Counter_Value"])
    ids = sorted(per)[-last:]
    names = sorted({n for i in ids for n in per[i]})
    return {n: statistics.mean(per[i][n] for i in ids if n in per[i]) for n in names}


def _counter_values(path: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter."""
    vals = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return vals


def _pick(vals, needle):
    hits = [v for k, v in vals.items() if needle in k]
    if not hits:
        raise SystemExit(f"no kernel matching {needle!r} in counter file")
    return [x for v in hits for x in v]


EA_COUNTERS = ("TCC_EA0_RDREQ_DRAM_32B_sum", "TCC_EA0_RDREQ_128B_sum", "TCC_EA0_RDREQ_64B_sum",
               "TCC_EA0_RDREQ_32B_sum")


def ea_reads(ea_csv: str, kernel: str, copy_mib: float) -> dict:
    """A second path to the read traffic: DRAM read requests counted in
    32-byte units (a 64-byte request counts 2, a 128-byte one 4), and the
    requests by size, per dispatch of the kernel and of the calibration
    copies.  Bytes = 32 x the DRAM count, with no scale factor; the copy shows
    whether that reading is exact."""
    vals = {c: _counter_values(ea_csv, c) for c in EA_COUNTERS}
    copy_bytes = copy_mib * 2 ** 20
    dram_k = statistics.mean(_pick(vals[EA_COUNTERS[0]], kernel)) * 32.0
    copies = [v * 32.0 for v in _pick(vals[EA_COUNTERS[0]], COPY_KERNEL_HINT)
              if copy_bytes / 4 <= v * 32.0 <= copy_bytes * 4]
    if not copies:
        raise SystemExit("no calibration copy found in the EA counter file")
    by_size = {c: statistics.mean(_pick(vals[c], kernel)) for c in EA_COUNTERS[1:]}
    sized = 128 * by_size[EA_COUNTERS[1]] + 64 * by_size[EA_COUNTERS[2]] + 32 * by_size[EA_COUNTERS[3]]
    return {"ea_read_bytes_per_launch": dram_k, "ea_copy_read_bytes": statistics.mean(copies),
            "ea_copy_scale": copy_bytes / statistics.mean(copies), "ea_requests_by_size": by_size,
            "ea_sized_read_bytes_per_launch": sized}


def traffic(fetch_csv: str, write_csv: str, kernel: str, copy_mib: float, workload: str) -> dict:
    fetch, write = _counter_values(fetch_csv, "FETCH_SIZE"), _counter_values(write_csv, "WRITE_SIZE")
    k_fetch, k_write = _pick(fetch, kernel), _pick(write, kernel)
    copy_bytes = copy_mib * 2 ** 20

    def calib(vals):
        # the calibration copies are the copy dispatches whose counter is
        # within a factor 4 of the copy size (setup copies are far smaller)
        kib = copy_bytes / 1024.0
        hits = [v for v in _pick(vals, COPY_KERNEL_HINT) if kib / 4 <= v <= kib * 4]
        if not hits:
            raise SystemExit("no calibration copy found in counter file")
        return statistics.mean(hits) * 1024.0

    s_fetch, s_write = copy_bytes / calib(fetch), copy_bytes / calib(write)
    fb = statistics.mean(k_fetch) * 1024.0 * s_fetch
    wb = statistics.mean(k_write) * 1024.0 * s_write
    return {"kernel": kernel, "workload": workload, "kernel_source_sha": kernel_source_hash(),
            "dispatches": len(k_fetch), "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
            "hbm_bytes_per_launch": fb + wb, "copy_calibration_bytes": copy_bytes,
            "fetch_scale": s_fetch, "write_scale": s_write}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("--top", type=int, default=12)
    l = sub.add_parser("last")
    l.add_argument("csv", help="kernel_trace.csv")
    l.add_argument("--kernel", default="k_split")
    l.add_argument("--n", type=int, default=36, help="dispatches at the end of the run (timed + back-to-back)")
    l.add_argument("--skip", type=int, default=0,
                   help="leave out this many dispatches at the very end (bench.py's single-launch timings)")
    se = sub.add_parser("series")
    se.add_argument("csv", help="kernel_trace.csv")
    se.add_argument("--kernel", default="k_split")
    se.add_argument("--first", type=int, default=300, help="dispatches from the start of the run")
    se.add_argument("--bin", type=int, default=10, help="dispatches per row")
    ck = sub.add_parser("clock")
    ck.add_argument("trace", help="kernel_trace.csv of a run that also collected GRBM_GUI_ACTIVE")
    ck.add_argument("counters", help="counter_collection.csv of the same run")
    ck.add_argument("--kernel", default="k_split")
    ck.add_argument("--bin", type=int, default=20)
    c = sub.add_parser("counters")
    c.add_argument("csv", help="counter_collection.csv")
    c.add_argument("--kernel", default="k_split")
    c.add_argument("--n", type=int, default=8, help="dispatches at the end of the run")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", default="k_split")
    t.add_argument("--copy-mib", type=float, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--ea", help="counter_collection.csv of the TCC_EA read-request counters (cross-check)")
    t.add_argument("--out")
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        print(stats_table(args.csv, args.top))
    elif args.cmd == "series":
        bins, total = dispatch_series(args.csv, args.kernel, args.first, args.bin)
        print(f"{args.kernel}: first {min(args.first, total)} of {total} dispatches, in start order")
        print("| dispatches | mean us | min us | max us |")
        print("|---|---|---|---|")
        for i0, i1, m, lo, hi in bins:
            print(f"| {i0}-{i1} | {m:.1f} | {lo:.1f} | {hi:.1f} |")
    elif args.cmd == "clock":
        print("| dispatches | mean us | clock GHz |")
        print("|---|---|---|")
        for i0, i1, d, g in clock_series(args.trace, args.counters, args.kernel, args.bin):
            print(f"| {i0}-{i1} | {d:.1f} | {g:.2f} |")
    elif args.cmd == "counters":
        for n, v in counter_means(args.csv, args.kernel, args.n).items():
            print(f"{n}: {v:.6g}")
    elif args.cmd == "last":
        mean, lo, hi, total = last_dispatches(args.csv, args.kernel, args.n, args.skip)
        where = f"last {args.n}" + (f" before the final {args.skip}" if args.skip else "")
        print(f"{args.kernel}: {where} of {total} dispatches: mean {mean:.2f} us, min {lo:.2f}, max {hi:.2f}")
    else:
        res = traffic(args.fetch, args.write, args.kernel, args.copy_mib, args.workload)
        if args.ea:
            res["cross_check"] = ea_reads(args.ea, args.kernel, args.copy_mib)
        txt = json.dumps(res, indent=1)
        if args.out:
            with open(args.out, "w") as f:
                f.write(txt + "\n")
        print(txt)


if __name__ == "__main__":
    sys.exit(main())
