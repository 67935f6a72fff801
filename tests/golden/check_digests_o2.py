"""Re-derive every stored full-size digest with the C++ oracle tier (oracle/ks_o2.cpp).

tests/golden/digests_full.json was written by the numpy oracle. This script
rebuilds every case's inputs from tests/golden/cases.py, key-switches every
(key, ciphertext) item with the C++ tier, which shares no code with the numpy
oracle, and compares each output digest with the stored one. It writes
nothing; it exits 1 on the first disagreement. The CPU tests run a sample of
the same comparison on every run.

Run from the repository root:  python tests/golden/check_digests_o2.py
(about two minutes on 8 cores).
"""

from __future__ import annotations

import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

import cases  # noqa: E402
from oracle import o2  # noqa: E402


def main() -> int:
    t0 = time.time()
    doc = cases.load_digests()
    total = 0
    for name, fn in cases.builders().items():
        made = fn()
        for c in (made if isinstance(made, tuple) else (made,)):
            O = o2.O2(c.prm.log2n, c.prm.L, c.prm.dnum, c.prm.K, c.prm.partition)
            want = doc["cases"][c.name]["digests"]
            got = {}
            if c.name == "n17_chain":
                relin, rot = c.keys
                for b in range(c.batch):
                    s1 = O.keyswitch(c.cts[b], c.level, relin.galois, relin.b, seed=relin.seed)
                    s2 = O.keyswitch(s1, c.level, rot.galois, rot.b, seed=rot.seed)
                    got[b], got[c.batch + b] = cases.digest(s1), cases.digest(s2)
            else:
                for r, k in enumerate(c.keys):
                    for b in range(c.batch):
                        y = O.keyswitch(c.cts[b], c.level, k.galois, k.b, seed=k.seed, evk_a=k.a)
                        got[r * c.batch + b] = cases.digest(y)
            bad = [i for i in range(len(want)) if got.get(i) != want[i]]
            total += len(want)
            print(f"[{time.time() - t0:6.0f} s] {c.name}: {len(want) - len(bad)}/{len(want)} digests agree",
                  flush=True)
            if bad:
                print(f"{c.name}: items {bad} differ from the stored digests", flush=True)
                return 1
            O.close()
    print(f"all {total} stored digests re-derived by the C++ oracle in {time.time() - t0:.0f} s", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
