"""Summaries of rocprofv3 output for the key-switching kernels.

Two subcommands turn rocprofv3 CSV files into the short text summaries kept
under profiles/ (each summary records the commands that produced it):

* ``stats``   from ``--kernel-trace --stats --output-format csv``: for every
  kernel family of the N=2^16, L=24, k=8 key switch (regenerated key half)
  and of the homomorphic multiplication of 8 pairs and the 4 x 4 linear
  transform around it, the average
  duration over the dispatches of that family's batch-8 launch, plus the
  kernel_stats table of the whole run.
* ``traffic`` from two ``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs of
  ``bench.py --calibrate-copy``: the counters of every family per dispatch,
  scaled by what the same counters read for a plain copy kernel of known size
  (an elementwise pass src -> dst over 256 MiB, launched by
  ``bench.py --calibrate-copy``), giving HBM bytes per launch.

A family's k=8 launch is the dispatch of its kernel with the largest grid in
the run (bench.py runs batch 8 and batch 1; within a family the batch-8
launch has the largest grid). The traffic summary also records a hash of the
device sources; bench.py reports a traffic figure only while the sources
still hash the same.

Usage:
  python -m key_switching_amd.profiling stats --trace T.csv --stats S.csv --cmd "..."
  python -m key_switching_amd.profiling traffic --fetch F.csv --write W.csv --cmd "..."
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

# kernel family (the names bench.py and the library's profiling API use) ->
# dispatch-name prefix of its launch in the N=2^16 key switch with a
# regenerated key half (the inner product at batch 8 is the producer/consumer
# kernel)
FAMILIES = {
    "modup_inv_blk": "k_modup_inv_blk<16>",
    "modup_inv_col": "k_modup_inv_col<16>",
    "modup_bconv": "k_modup_bconv<16, 6, 3>",
    "modup_fwd_blk": "k_modup_fwd_blk<16>",
    "inner_product": "k_ip_regen<4, 12, 8, false>",
    "moddown_inv_blk": "k_md_inv_blk<16>",
    "moddown_inv_col": "k_md_inv_col<16>",
    "moddown_bconv": "k_md_bconv<16, 6, 3>",
    "moddown_fwd_blk": "k_md_fwd_blk<16, false, false>",
    # homomorphic multiplication of 8 pairs around the same key switch
    "tensor": "k_tensor",
    "rescale_gather": "k_rs_gather",
    "rescale_col": "k_rs_col<16>",
    "moddown_rescale": "k_md_rs_blk<16, false>",
    # the 4 x 4 double-hoisted linear transform of one ciphertext
    "bsgs_baby": "k_bsgs_baby<4>",
    "bsgs_giant": "k_bsgs_giant",
}


def device_source_hash() -> str:
    h = hashlib.sha256()
    for rel in DEVICE_SOURCES:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    return name.split("(")[0].replace("void ", "").replace("pc::", "").strip()


def _grid(row: dict) -> int:
    """Total work-items of a dispatch (counter CSVs give Grid_Size, traces X, Y and Z)."""
    if row.get("Grid_Size", "") != "":
        return int(row["Grid_Size"])
    return int(row.get("Grid_Size_X", 1)) * int(row.get("Grid_Size_Y", 1)) * int(row.get("Grid_Size_Z", 1))


def _family_rows(rows, prefix):
    mine = [r for r in rows if _short(r["Kernel_Name"]) == prefix]
    if not mine:
        return [], 0
    g = max(_grid(r) for r in mine)
    return [r for r in mine if _grid(r) == g], g


def cmd_stats(a) -> str:
    rows = list(csv.DictReader(open(a.trace)))
    out = [f"# rocprofv3 kernel statistics: {a.title}", "",
           "Commands:", "", "```", a.cmd, "```", "",
           f"device_sources_hash: {device_source_hash()}", ""]
    if a.note:
        out += [a.note, ""]
    out += ["Per kernel family, dispatches of its batch-8 launch (largest grid of that kernel in the run):", "",
           "| family | dispatch | grid | launches | avg us | median us | min us | max us |",
           "|---|---|---|---|---|---|---|---|"]
    for fam, prefix in FAMILIES.items():
        sel, g = _family_rows(rows, prefix)
        if not sel:
            continue
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in sel]
        out.append(f"| {fam} | `{prefix}` | {g} | {len(d)} | {statistics.mean(d):.2f} | "
                   f"{statistics.median(d):.2f} | {min(d):.2f} | {max(d):.2f} |")
    out += ["", "kernel_stats.csv (all dispatches of the run, every batch size):", "", "```"]
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
        key = (r["Dispatch_Id"], _short(r["Kernel_Name"]), _grid(r))
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return per


def cmd_traffic(a) -> str:
    f = _counter_per_dispatch(a.fetch, "FETCH_SIZE")
    w = _counter_per_dispatch(a.write, "WRITE_SIZE")
    cf = [v for (d, k, g), v in f.items() if COPY_KERNEL_HINT in k.lower()]
    cw = [v for (d, k, g), v in w.items() if COPY_KERNEL_HINT in k.lower()]
    if not cf or not cw:
        raise SystemExit("no copy-kernel dispatches in the counter files")
    cf_big, cw_big = max(cf), max(cw)
    rf = COPY_BYTES / (cf_big * 1024.0)
    rw = COPY_BYTES / (cw_big * 1024.0)
    out = [f"# HBM traffic per launch: {a.title}", "",
           "Commands:", "", "```", a.cmd, "```", "",
           f"device_sources_hash: {device_source_hash()}",
           f"copy calibration: plain copy of {COPY_BYTES} bytes read FETCH_SIZE {cf_big:.0f} KiB, "
           f"WRITE_SIZE {cw_big:.0f} KiB -> scale read {rf:.4f}, write {rw:.4f}", "",
           "Per kernel family, batch-8 launch (largest grid of that kernel), medians over its dispatches:", "",
           "| family | dispatch | grid | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | fetch bytes | write bytes | traffic bytes |",
           "|---|---|---|---|---|---|---|---|---|"]
    for fam, prefix in FAMILIES.items():
        fk = {(d, g): v for (d, k, g), v in f.items() if k == prefix}
        wk = {(d, g): v for (d, k, g), v in w.items() if k == prefix}
        if not fk or not wk:
            continue
        g = max(gg for (_, gg) in fk)
        kf = [v for (d, gg), v in fk.items() if gg == g]
        kw = [v for (d, gg), v in wk.items() if gg == g]
        fb = statistics.median(kf) * 1024.0 * rf
        wb = statistics.median(kw) * 1024.0 * rw
        out.append(f"| {fam} | `{prefix}` | {g} | {len(kf)} | {statistics.median(kf):.0f} | "
                   f"{statistics.median(kw):.0f} | {fb:.0f} | {wb:.0f} | {fb + wb:.0f} |")
    return "\n".join(out) + "\n"


def read_traffic(path: str, family: str):
    """Traffic bytes per launch of a family from a traffic summary, or None if absent or stale."""
    if not os.path.exists(path):
        return None
    text = open(path).read().splitlines()
    hash_ok = any(line.strip() == f"device_sources_hash: {device_source_hash()}" for line in text)
    if not hash_ok:
        return None
    for line in text:
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 9 and cells[0] == family:
            try:
                return float(cells[8])
            except ValueError:
                return None
    return None


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--trace", required=True)
    s.add_argument("--stats", required=True)
    s.add_argument("--top", type=int, default=24)
    s.add_argument("--title", default="")
    s.add_argument("--cmd", default="")
    s.add_argument("--note", default="")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--title", default="")
    t.add_argument("--cmd", default="")
    a = ap.parse_args(argv)
    sys.stdout.write(cmd_stats(a) if a.cmd_name == "stats" else cmd_traffic(a))


if __name__ == "__main__":
    main()
