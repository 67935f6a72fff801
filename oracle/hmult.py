"""Homomorphic multiplication around the key switch (oracle; test infrastructure only).

The pages name the product whose relinearisation the key switch performs
(Perseus README, 'What's inside': the session's ops, among them squaring a
ciphertext) but do not write it down. This module follows the textbook RNS-CKKS
multiplication, step by step, for ciphertexts a = (a0, a1), b = (b0, b1) at
level l in evaluation form:

1. Tensor product, limb by limb and position by position:
   d0 = a0 b0, d1 = a0 b1 + a1 b0, d2 = a1 b1 (mod q_i).
2. Relinearisation of d2 with the key for s^2: the key switch of (d0, d2)
   gives (d0 + KS_0(d2), KS_1(d2)); d1 is added to the second component.
3. Rescale by the last prime q_{l-1}, rounded: with x the coefficients of
   limb l-1 taken to (-q_{l-1}/2, q_{l-1}/2], every other limb becomes
   (c_i - NTT_i(x mod q_i)) * q_{l-1}^-1 mod q_i. Per coefficient this is
   round(C / q_{l-1}) mod q_i for C the integer with residues c_i.

The rounding reading (the centred residue, which is round-half-away for the odd
prime q_{l-1}) is listed in the design notes.
"""

from __future__ import annotations

import numpy as np

from . import keyswitch as ks
from .rns import centered, intt, ntt

U64 = np.uint64


def tensor(prm: ks.Params, a: np.ndarray, b: np.ndarray, level: int) -> np.ndarray:
    """d [3][l][N] = (a0 b0, a0 b1 + a1 b0, a1 b1) per limb (evaluation form)."""
    a = np.asarray(a, dtype=U64)
    b = np.asarray(b, dtype=U64)
    d = np.empty((3, level, prm.N), dtype=U64)
    for i in range(level):
        q = U64(prm.q[i])
        d[0, i] = a[0, i] * b[0, i] % q
        d[1, i] = (a[0, i] * b[1, i] % q + a[1, i] * b[0, i] % q) % q
        d[2, i] = a[1, i] * b[1, i] % q
    return d


def rescale(prm: ks.Params, ct: np.ndarray, level: int) -> np.ndarray:
    """[2][l][N] -> [2][l-1][N]: divide by q_{l-1}, rounding to nearest."""
    if level < 2:
        raise ValueError("rescale needs at least two primes")
    ct = np.asarray(ct, dtype=U64)
    ql = prm.q[level - 1]
    out = np.empty((ct.shape[0], level - 1, prm.N), dtype=U64)
    for u in range(ct.shape[0]):
        x = centered(intt(ct[u, level - 1], ql), ql)  # in (-q/2, q/2]
        for i in range(level - 1):
            q = prm.q[i]
            xi = ntt((x % q).astype(U64), q)
            diff = (ct[u, i] + (U64(q) - xi)) % U64(q)
            out[u, i] = diff * U64(pow(ql, -1, q)) % U64(q)
    return out


def relinearise(prm: ks.Params, d: np.ndarray, key: ks.Key, level: int) -> np.ndarray:
    """(d0 + KS_0(d2), d1 + KS_1(d2)) for the key of s^2."""
    if key.galois != 1:
        raise ValueError("relinearisation needs the key of s^2 (Galois element 1)")
    out = ks.keyswitch(prm, np.stack([d[0], d[2]]), key, level)
    for i in range(level):
        out[1, i] = (out[1, i] + d[1, i]) % U64(prm.q[i])
    return out


def hmult(prm: ks.Params, a: np.ndarray, b: np.ndarray, key: ks.Key, level: int) -> np.ndarray:
    """Tensor, relinearise, rescale: [2][l-1][N]."""
    return rescale(prm, relinearise(prm, tensor(prm, a, b, level), key, level), level)
