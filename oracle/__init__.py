"""CPU oracle for CKKS hybrid key switching (test infrastructure only).

This package is the checker for the GPU library, not part of it. Only the
tests, the smoke check and the benchmark's CPU-baseline leg may import it; the
GPU library never calls it and shares no code, constants or tables with it.

Everything here is plain numpy (uint64 holding values below 2^62) and Python
integers, written for a reader who checks it against the definitions:

* ``rns``       NTT-friendly primes, the negacyclic root psi, the negacyclic
                NTT as its definition a_hat[j] = a(psi^(2j+1)) evaluated with a
                textbook radix-2 FFT, and its inverse.
* ``chacha``    the ChaCha block function with the round count as a parameter
                and the seed expander that regenerates a key's uniform half.
* ``keyswitch`` parameters, digit partition, ModUp, automorphism, inner
                product, ModDown, key switch (single, batched, hoisted),
                key generation and the decryption check with its error bound.

A second tier, ``ks_o2.cpp`` (plain C++17 with OpenMP, loaded through
``o2``), computes the same key switch from the same definitions with its own
primes, roots, NTT and ChaCha, sharing no code with the numpy modules. The
tests compare the two word for word, at small and full sizes; the benchmark
times the C++ tier as its CPU baseline.

Source of the method: the Perseus README ('What's inside': the GPU re-creates
one half of each key-switching key from a ChaCha12 seed; 'Layout':
the runtime's NTT and key-switching kernels) and the arXiv summary page of the
Perseus paper (methodology item (i)). The pages do not spell out hybrid key
switching itself; every step here is the textbook RNS-CKKS algorithm under
the readings listed in the module docstrings.

Parity status: every function is pinned by tests under ``tests/`` against
definitions, closed forms, invariants or library routines (sympy, the OpenSSL
command line); ChaCha at 12 rounds is pinned only through the same
round-parameterised code being OpenSSL-exact at 20 rounds.
"""
