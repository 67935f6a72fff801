"""Write tests/golden/digests_full.json: the oracle's output digests of the full-size cases.

Calls only oracle/ and the input recipe in tests/golden/cases.py (which draws
from ks_inputs). Every (key, ciphertext) item of every case is key-switched by
the oracle and the SHA-256 of its output words is stored; the GPU parity tests
rebuild the inputs and compare the digest of every output item. The file also
records a hash of the sources the digests depend on (oracle/, ks_inputs.py,
cases.py), which a CPU test checks, so a change there cannot leave stale
digests behind.

Run from the repository root:  python tests/golden/make_digests.py [--jobs 8]
(about 15 minutes of CPU time; N=2^17 key switches take about 45 s each).
"""

from __future__ import annotations

import argparse
import json
import multiprocessing as mp
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

import cases  # noqa: E402
from oracle import keyswitch as ks  # noqa: E402

_CASES = {}  # built in the parent before the workers fork


def _build_all():
    for name, fn in cases.builders().items():
        made = fn()
        for c in (made if isinstance(made, tuple) else (made,)):
            _CASES[c.name] = c


def _tasks():
    """(cost, case name, task argument); the most expensive first."""
    out = []
    for b in range(8):
        out.append((90, "n17_chain", b))
    for b in range(8):
        out.append((2, "n16_relin_k8", b))
        out.append((2, "n16_extreme_x", b))
        out.append((2, "n16_extreme_y", b))
    for t in range(4):
        out.append((5, "n16_hoist16", t))
    for level in cases.LEVELS:
        for b in range(8):
            out.append((level / 12.0, f"n16_level{level}", b))
    return sorted(out, key=lambda x: -x[0])


def _run(task):
    _, name, arg = task
    c = _CASES[name]
    res = []
    if name == "n17_chain":
        relin, rot = c.keys
        step1 = ks.keyswitch(c.prm, c.cts[arg], relin, c.level)
        step2 = ks.keyswitch(c.prm, step1, rot, c.level)
        res = [(arg, cases.digest(step1)), (8 + arg, cases.digest(step2))]
    elif name == "n16_hoist16":
        keys = c.keys[4 * arg: 4 * arg + 4]
        outs = ks.keyswitch_hoisted(c.prm, c.cts[0], keys, c.level)
        res = [(4 * arg + k, cases.digest(o)) for k, o in enumerate(outs)]
    else:
        outs = ks.keyswitch_hoisted(c.prm, c.cts[arg], c.keys, c.level)
        res = [(r * c.batch + arg, cases.digest(o)) for r, o in enumerate(outs)]
    return name, res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    args = ap.parse_args()
    t0 = time.time()
    _build_all()
    print(f"inputs built in {time.time() - t0:.0f} s", flush=True)
    digests = {name: [None] * (len(c.keys) * c.batch) for name, c in _CASES.items()}
    with mp.get_context("fork").Pool(args.jobs) as pool:
        for name, res in pool.imap_unordered(_run, _tasks()):
            for idx, d in res:
                digests[name][idx] = d
            print(f"[{time.time() - t0:6.0f} s] {name}: {len(res)} digests", flush=True)
    doc = {"sources_hash": cases.sources_hash(),
           "digest": "SHA-256 of each output's [2][l][N] words as little-endian uint32",
           "writer": "tests/golden/make_digests.py (oracle/ only; inputs from tests/golden/cases.py)",
           "cases": {}}
    for name, c in sorted(_CASES.items()):
        assert all(d is not None for d in digests[name]), name
        entry = {"log2n": c.prm.log2n, "L": c.prm.L, "dnum": c.prm.dnum, "K": c.prm.K, "level": c.level,
                 "batch": c.batch, "galois": [k.galois for k in c.keys], "stored_a": c.stored,
                 "digests": digests[name]}
        if name == "n17_chain":
            entry["order"] = "items 0..7 after relinearisation, then items 0..7 after the X^5 rotation"
        else:
            entry["order"] = "index = key * batch + ciphertext"
        doc["cases"][name] = entry
    with open(cases.DIGEST_FILE, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(f"wrote {cases.DIGEST_FILE} in {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main()
