"""Summaries of rocprofv3 output for the key-switching kernels.

Two subcommands turn rocprofv3 CSV files into the short text summaries kept
under profiles/ (each summary records the commands that produced it):

* ``stats``   from ``--kernel-trace --stats --output-format csv``: the
  kernel_stats table, plus the average duration of one kernel over only the
  dispatches with a given grid size (the bench runs several batch sizes, so a
  per-name average would mix them).
* ``traffic`` from two ``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs of
  ``bench.py --calibrate-copy``: the counters of one kernel per dispatch,
  scaled by what the same counters read for a plain copy kernel of known size
  (an elementwise pass src -> dst over 256 MiB, launched by
  ``bench.py --calibrate-copy``), giving HBM bytes per launch.

The traffic summary also records a hash of the device sources; bench.py
reports the traffic figure only while the sources still hash the same.

Usage:
  python -m key_switching_amd.profiling stats --trace T.csv --stats S.csv --kernel NAME --family F --grid G --cmd "..."
  python -m key_switching_amd.profiling traffic --fetch F.csv --write W.csv --kernel NAME --family F --grid G --cmd "..."
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
DEVICE_SOURCES = ("csrc/kernels.hip", "csrc/ntt_pass.h", "csrc/device_common.h")
COPY_BYTES = 256 << 20
COPY_KERNEL_HINT = "elementwise"  # bench.py --calibrate-copy: torch.bitwise_or(src, 0, out=dst)


def device_source_hash() -> str:
    h = hashlib.sha256()
    for rel in DEVICE_SOURCES:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    return name.split("(")[0].replace("void ", "").strip()


def _grid(row: dict) -> int:
    """Total work-items of a dispatch (counter CSVs give Grid_Size, traces X, Y and Z)."""
    if row.get("Grid_Size", "") != "":
        return int(row["Grid_Size"])
    return int(row.get("Grid_Size_X", 1)) * int(row.get("Grid_Size_Y", 1)) * int(row.get("Grid_Size_Z", 1))


def cmd_stats(a) -> str:
    rows = list(csv.DictReader(open(a.trace)))
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows
            if a.kernel in r["Kernel_Name"] and _grid(r) == a.grid]
    out = [f"# rocprofv3 kernel statistics: {a.title}", "",
           "Commands:", "", "```", a.cmd, "```", "",
           f"Device sources hash: {device_source_hash()}", ""]
    if durs:
        out += [f"Kernel family `{a.family}` (dispatches named `{a.kernel}`, grid size {a.grid}): {len(durs)} launches, "
                f"average {statistics.mean(durs):.2f} us, median {statistics.median(durs):.2f} us, "
                f"min {min(durs):.2f} us, max {max(durs):.2f} us", ""]
    out += ["kernel_stats.csv (all dispatches of the run, every batch size):", "", "```"]
    srows = list(csv.DictReader(open(a.stats)))
    keys = [k for k in ("Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage") if k in srows[0]]
    out.append(" | ".join(keys))
    for r in srows[: a.top]:
        out.append(" | ".join(_short(r[k]) if k == "Name" else r[k] for k in keys))
    out.append("```")
    return "\n".join(out) + "\n"


def _counter_per_dispatch(path: str, counter: str):
    per = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        key = (r["Dispatch_Id"], r["Kernel_Name"], _grid(r))
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return per


def cmd_traffic(a) -> str:
    f = _counter_per_dispatch(a.fetch, "FETCH_SIZE")
    w = _counter_per_dispatch(a.write, "WRITE_SIZE")

    def kernel_vals(per, name, grid=None):
        return [v for (d, k, g), v in per.items() if name in k and (grid is None or g == grid)]

    cf = [v for (d, k, g), v in f.items() if COPY_KERNEL_HINT in k.lower()]
    cw = [v for (d, k, g), v in w.items() if COPY_KERNEL_HINT in k.lower()]
    cf_big = max(cf) if cf else None
    cw_big = max(cw) if cw else None
    kf = kernel_vals(f, a.kernel, a.grid)
    kw = kernel_vals(w, a.kernel, a.grid)
    if not (cf_big and cw_big and kf and kw):
        raise SystemExit("missing copy or kernel dispatches in the counter files")
    rf = COPY_BYTES / (cf_big * 1024.0)
    rw = COPY_BYTES / (cw_big * 1024.0)
    fetch_b = statistics.median(kf) * 1024.0 * rf
    write_b = statistics.median(kw) * 1024.0 * rw
    out = [f"# HBM traffic per launch: {a.title}", "",
           "Commands:", "", "```", a.cmd, "```", "",
           f"device_sources_hash: {device_source_hash()}",
           f"kernel: {a.family}",
           f"dispatch_filter: {a.kernel}",
           f"grid_size: {a.grid}",
           f"copy calibration: plain copy of {COPY_BYTES} bytes read FETCH_SIZE {cf_big:.0f} KiB, "
           f"WRITE_SIZE {cw_big:.0f} KiB -> scale read {rf:.4f}, write {rw:.4f}",
           f"kernel dispatches: {len(kf)} (FETCH_SIZE), {len(kw)} (WRITE_SIZE); medians "
           f"{statistics.median(kf):.0f} KiB fetched, {statistics.median(kw):.0f} KiB written",
           f"fetch_bytes_per_launch: {fetch_b:.0f}",
           f"write_bytes_per_launch: {write_b:.0f}",
           f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}", ""]
    return "\n".join(out)


def read_traffic(path: str, kernel: str):
    """Traffic bytes per launch from a traffic summary, or None if absent or stale."""
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel") != kernel or vals.get("device_sources_hash") != device_source_hash():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--trace", required=True)
    s.add_argument("--stats", required=True)
    s.add_argument("--kernel", required=True, help="substring of the dispatch name")
    s.add_argument("--family", required=True, help="kernel family name used by bench.py")
    s.add_argument("--grid", type=int, required=True)
    s.add_argument("--top", type=int, default=16)
    s.add_argument("--title", default="")
    s.add_argument("--cmd", default="")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True, help="substring of the dispatch name")
    t.add_argument("--family", required=True, help="kernel family name used by bench.py")
    t.add_argument("--grid", type=int, required=True)
    t.add_argument("--title", default="")
    t.add_argument("--cmd", default="")
    a = ap.parse_args(argv)
    sys.stdout.write(cmd_stats(a) if a.cmd_name == "stats" else cmd_traffic(a))


if __name__ == "__main__":
    main()
