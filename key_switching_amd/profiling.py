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
    # the relinearisation key (Galois element 1): block pass and inner product fused
    "modup_ip": "k_modup_ip<16, 4, 12, false>",
    "moddown_inv_blk": "k_md_inv_blk<16>",
    "moddown_inv_col": "k_md_inv_col<16>",
    "moddown_bconv": "k_md_bconv<16, 6, 3>",
    "moddown_fwd_blk": "k_md_fwd_blk<16, 1, false>",
    # homomorphic multiplication of 8 pairs around the same key switch
    "tensor": "k_tensor",
    "rescale_gather": "k_rs_gather",
    "rescale_col": "k_rs_col<16>",
    "moddown_rescale": "k_md_rs_blk<16, false>",
    # the 4 x 4 double-hoisted linear transform of one ciphertext
    "bsgs_baby": "k_bsgs_baby<4>",
    "bsgs_giant": "k_bsgs_giant",
}


# the N=2^17, L=40 chain (bench.py --only n17): batch-8 launches, a half
# regenerated or stored. Each chain call relinearises (the fused block pass
# and inner product), then rotates (block pass to ext, then the gathering
# inner product). A (prefix, parity) entry would take every other dispatch of
# a kernel in dispatch order, for two steps that run the same kernel.
FAMILIES_N17 = {
    "modup_bconv": "k_modup_bconv<17, 8, 3>",
    # relinearisation step: the fused block pass and inner product; rotation
    # step: the block pass to ext, then the gathering inner product
    "modup_ip_chacha_relin": "k_modup_ip<17, 5, 12, false>",
    "modup_ip_stored_relin": "k_modup_ip<17, 5, 12, true>",
    "modup_fwd_blk_rotate": "k_modup_fwd_blk<17>",
    "inner_product_chacha_rotate": "k_inner_product<5, 12, false, 8, false>",
    "inner_product_stored_rotate": "k_inner_product<5, 12, true, 8, false>",
    "moddown_bconv": "k_md_bconv<17, 8, 3>",
    "moddown_fwd_blk_relin": "k_md_fwd_blk<17, 1, false>",
    "moddown_fwd_blk_rotate": "k_md_fwd_blk<17, 2, true>",
}
FAMILY_SETS = {"n16": FAMILIES, "n17": FAMILIES_N17}

# Kernels whose grid does not grow with the batch (the fused tile loops over
# the items): a dispatch is the family's batch-8 launch when the dispatch just
# before it on its queue is the batch-8 launch (largest grid) of the kernel
# named here, the one that precedes it in every key switch.
FOLLOWS = {"k_modup_ip<16, 4, 12, false>": "k_modup_bconv<16, 6, 3>"}


def _batch8_ids(disp, prefix):
    """Dispatch ids of the batch-8 launch of `prefix` and its grid. disp maps a
    dispatch id (int) to (queue, short kernel name, grid)."""
    mine = [d for d, (_, k, _) in disp.items() if k == prefix]
    if not mine:
        return [], 0
    g = max(disp[d][2] for d in mine)
    if prefix not in FOLLOWS:
        return sorted(d for d in mine if disp[d][2] == g), g
    pred = FOLLOWS[prefix]
    pg = max((gg for (_, k, gg) in disp.values() if k == pred), default=-1)
    prev, out = {}, []
    for d in sorted(disp):
        q, k, gg = disp[d]
        if k == prefix and q in prev and prev[q] == (pred, pg):
            out.append(d)
        prev[q] = (k, gg)
    return out, g


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
    disp = {int(r["Dispatch_Id"]): (r.get("Queue_Id", ""), _short(r["Kernel_Name"]), _grid(r)) for r in rows}
    ids, g = _batch8_ids(disp, prefix)
    keep = set(ids)
    return [r for r in rows if int(r["Dispatch_Id"]) in keep], g


def cmd_stats(a) -> str:
    rows = list(csv.DictReader(open(a.trace)))
    out = [f"# rocprofv3 kernel statistics: {a.title}", "",
           "Commands:", "", "```", a.cmd, "```", "",
           f"device_sources_hash: {device_source_hash()}", ""]
    if a.note:
        out += [a.note, ""]
    out += ["Per kernel family, dispatches of its batch-8 launch (largest grid of that kernel in the run; for "
            "the fused tile, whose grid does not grow with the batch, the dispatches that follow a batch-8 "
            "base conversion):", "",
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
    """Counter value per dispatch, keyed (dispatch id, short name, grid), and the
    dispatch table (id -> queue, short name, grid) of the file."""
    per, disp = {}, {}
    for r in csv.DictReader(open(path)):
        disp[int(r["Dispatch_Id"])] = (r.get("Queue_Id", ""), _short(r["Kernel_Name"]), _grid(r))
        if r["Counter_Name"] != counter:
            continue
        key = (r["Dispatch_Id"], _short(r["Kernel_Name"]), _grid(r))
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return per, disp


def cmd_traffic(a) -> str:
    f, fdisp = _counter_per_dispatch(a.fetch, "FETCH_SIZE")
    w, wdisp = _counter_per_dispatch(a.write, "WRITE_SIZE")
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
    for fam, spec in FAMILY_SETS[a.families].items():
        prefix, parity = (spec, None) if isinstance(spec, str) else spec
        fk = {(d, g): v for (d, k, g), v in f.items() if k == prefix}
        wk = {(d, g): v for (d, k, g), v in w.items() if k == prefix}
        if not fk or not wk:
            continue
        g = max(gg for (_, gg) in fk)

        def pick(m, disp):
            ids, _ = _batch8_ids(disp, prefix)
            ds = [str(d) for d in ids if (str(d), g) in m]
            if parity is not None:
                ds = ds[parity::2]
            return [m[(d, g)] for d in ds]

        kf, kw = pick(fk, fdisp), pick(wk, wdisp)
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


def read_valu_ratio(path: str, family: str):
    """Issued VALU lane-operations over the model's algorithmic operations for one
    family, from a VALU summary (None if absent or stale)."""
    if not os.path.exists(path):
        return None
    text = open(path).read().splitlines()
    if not any(line.strip() == f"device_sources_hash: {device_source_hash()}" for line in text):
        return None
    for line in text:
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 5 and cells[0] == family:
            try:
                return float(cells[4])
            except ValueError:
                return None
    return None


def read_ip_traffic(path: str):
    """Inner-product traffic per batch-8 launch of the N=2^17 chain (the fused launch
    for the relinearisation step), regenerated and stored a halves, from its
    traffic summary (None if absent or stale)."""
    if not os.path.exists(path):
        return None
    text = open(path).read().splitlines()
    if not any(line.strip() == f"device_sources_hash: {device_source_hash()}" for line in text):
        return None
    out = {}
    for line in text:
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 9 and cells[0].startswith(("inner_product_", "modup_ip_")):
            _, _, half, step = cells[0].split("_")
            out.setdefault(half, {})[step] = {"fetch": float(cells[6]), "write": float(cells[7]),
                                              "total": float(cells[8])}
    return out or None


# SQ counters of the VALU summary (one rocprofv3 pass: at most 8 SQ and 2 GRBM counters)
VALU_COUNTERS = ("SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU", "SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES",
                 "SQ_INSTS_LDS", "SQ_WAIT_INST_ANY", "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE")


def _per_dispatch(path: str):
    rows, meta = {}, {}
    for r in csv.DictReader(open(path)):
        d = int(r["Dispatch_Id"])
        rows.setdefault(d, {})[r["Counter_Name"]] = rows.get(d, {}).get(r["Counter_Name"], 0.0) + float(
            r["Counter_Value"])
        meta[d] = (_short(r["Kernel_Name"]), _grid(r), int(r.get("VGPR_Count", 0) or 0),
                   (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3, r["Kernel_Name"],
                   r.get("Queue_Id", ""))
    return rows, meta


def cmd_valu(a) -> str:
    """Issued VALU instructions per kernel family against the model's algorithmic
    int32 operations (bench.alg_ops at N=2^16, L=24, dnum=4, K=6, batch 8)."""
    sys.path.insert(0, os.path.dirname(HERE))
    import bench
    rows, meta = _per_dispatch(a.pmc)
    clock = bench.CLOCK_GHZ * 1e3  # MHz -> cycles per us
    simds = bench.CUS * 4
    out = [f"# VALU instruction counts: {a.title}", "", "Commands:", "", "```", a.cmd, "```", "",
           f"device_sources_hash: {device_source_hash()}", "",
           "Per kernel family, batch-8 launch (largest grid of that kernel), medians over its dispatches.",
           "`issued/alg` = SQ_INSTS_VALU x 64 lanes / the model's algorithmic int32 operations of the launch; "
           "`issue us` = SQ_INSTS_VALU x 4 cycles / 1024 SIMDs / 2.4 GHz, the launch's time if the VALU issued "
           "every cycle at the peak clock; `busy` = issue us / the launch's duration in this counter run "
           "(serialised dispatches); `wait` = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES; `bank` = "
           "SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS.", "",
           "| family | dispatch | grid | VALU wave-instr (M) | issued/alg | issue us | duration us | busy | "
           "LDS instr (M) | bank | wait |",
           "|---|---|---|---|---|---|---|---|---|---|---|"]
    N, L, K, alpha, beta, batch = 1 << 16, 24, 6, 6, 4, 8
    for fam, prefix in FAMILIES.items():
        if fam not in bench.KERNELS and fam != "modup_ip":
            continue
        ds, g = _batch8_ids({d: (m[5], m[0], m[1]) for d, m in meta.items()}, prefix)
        if not ds:
            continue

        def med(c):
            return statistics.median(rows[d].get(c, 0.0) for d in ds)

        valu = med("SQ_INSTS_VALU")
        alg = bench.alg_ops(fam, N, L, K, alpha, beta, batch)
        issue_us = valu * 4 / simds / clock
        dur = statistics.median(meta[d][3] for d in ds)
        lds = med("SQ_INSTS_LDS")
        out.append(f"| {fam} | `{prefix}` | {g} | {valu / 1e6:.2f} | {valu * 64 / alg:.3f} | {issue_us:.1f} | "
                   f"{dur:.1f} | {issue_us / dur:.2f} | {lds / 1e6:.2f} | "
                   f"{med('SQ_LDS_BANK_CONFLICT') / max(lds, 1):.3f} | "
                   f"{med('SQ_WAIT_INST_ANY') / max(med('SQ_WAVE_CYCLES'), 1):.2f} |")
    return "\n".join(out) + "\n"


PROBE_NAMES = {"0": "v_add_u32", "1": "v_mul_lo_u32", "2": "v_mul_hi_u32", "3": "v_mad_u64_u32", "4": "v_add3_u32",
               "5": "v_min_u32", "6": "v_xor_b32", "7": "v_alignbit_b32", "8": "butterfly (11 instructions)"}


def cmd_rates(a) -> str:
    """Issue rates of the instruction-rate probe (key_switching_amd/rate_probe) from a
    `rocprofv3 --pmc SQ_INSTS_VALU GRBM_GUI_ACTIVE` run. GRBM_GUI_ACTIVE is summed over
    the 8 XCDs, so GUI_ACTIVE / 8 / duration is the engine clock during the dispatch."""
    rows, meta = _per_dispatch(a.pmc)
    out = [f"# VALU issue rates of 32-bit integer instructions: {a.title}", "", "Commands:", "", "```", a.cmd,
           "```", "",
           "Each probe kernel runs 8 independent chains of one operation per thread (2048 workgroups of 256 "
           "threads, 4096 iterations); its loop body is that operation alone (checked in the gfx950 assembly "
           "of the build). `rate` = SQ_INSTS_VALU / (256 CUs x clock x duration), in wave-instructions per CU "
           "per clock; 1.0 is the four SIMD16s each issuing one wave64 instruction every 4 clocks. "
           "`clock` = GRBM_GUI_ACTIVE / 8 XCDs / duration.", "",
           "| instruction | dispatches | VALU wave-instr (M) | duration us | clock GHz | rate at 2.4 GHz | "
           "rate at the measured clock |", "|---|---|---|---|---|---|---|"]
    for op, name in PROBE_NAMES.items():
        ds = [d for d, m in meta.items() if f"k_probe<{op}>(" in m[4]]
        if not ds:
            continue
        valu = statistics.median(rows[d]["SQ_INSTS_VALU"] for d in ds)
        dur = statistics.median(meta[d][3] for d in ds)
        gui = statistics.median(rows[d]["GRBM_GUI_ACTIVE"] for d in ds)
        clk = gui / 8 / (dur * 1e3)
        out.append(f"| {name} | {len(ds)} | {valu / 1e6:.1f} | {dur:.1f} | {clk:.3f} | "
                   f"{valu / (256 * 2.4e3 * dur):.3f} | {valu / (256 * clk * 1e3 * dur):.3f} |")
    return "\n".join(out) + "\n"


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
    t.add_argument("--families", choices=sorted(FAMILY_SETS), default="n16")
    v = sub.add_parser("valu")
    v.add_argument("--pmc", required=True)
    v.add_argument("--title", default="")
    v.add_argument("--cmd", default="")
    q = sub.add_parser("rates")
    q.add_argument("--pmc", required=True)
    q.add_argument("--title", default="")
    q.add_argument("--cmd", default="")
    a = ap.parse_args(argv)
    fn = {"stats": cmd_stats, "traffic": cmd_traffic, "valu": cmd_valu, "rates": cmd_rates}[a.cmd_name]
    sys.stdout.write(fn(a))


if __name__ == "__main__":
    main()
