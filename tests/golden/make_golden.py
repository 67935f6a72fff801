"""Write the parameter fixtures of tests/golden from the oracle alone.

For each ring size used by the workloads, the fixture lists the prime chain
(every prime q < 2^31 with q = 1 mod 2N, descending: L ciphertext primes then
K special primes) and each prime's psi (the smallest primitive 2N-th root of
unity). These are the readings of the pages' "32-bit chain" taken by the
oracle; the library's host tables are compared with them on the CPU.

Run: python tests/golden/make_golden.py   (from the repository root)
"""

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import rns  # noqa: E402

CHAINS = {12: 4, 16: 30, 17: 48}


def main():
    for log2n, count in CHAINS.items():
        N = 1 << log2n
        primes = rns.ntt_primes(N, count)
        doc = {"log2n": log2n, "primes": primes, "psi": [rns.find_psi(p, N) for p in primes],
               "source": "oracle/rns.py via tests/golden/make_golden.py"}
        with open(os.path.join(HERE, f"chain_n{log2n}.json"), "w") as f:
            json.dump(doc, f, indent=1)
            f.write("\n")


if __name__ == "__main__":
    main()
