"""Seeded synthetic inputs for CKKS hybrid key switching.

This module is shared by the tests, the benchmark and the smoke check. It
holds workload shapes and random draws only: no NTT, no base conversion, no
key generation and no ChaCha. The primes a draw needs are passed in by the
caller, so neither the GPU library nor the CPU oracle depends on the other
through this file.

Workloads (synthetic, uniform by construction; the pages publish no test
vectors for key switching):

* ``tiny``     N=2^12, L=3, dnum=3 (alpha=1), K=1, one rotation key X->X^5,
               one ciphertext, ChaCha key seed all zeros.
* ``n16``      N=2^16, L=24, dnum=4 (alpha=6), K=6, relinearisation key,
               batches k=1 and k=8 (the headline workload).
* ``hoist16``  N=2^16, L=24, dnum=4, K=6, one ciphertext, 16 rotation keys
               X->X^(5^r) r=1..16 applied after one shared ModUp.
* ``levels16`` N=2^16, levels 24,20,16,12,8,4, alpha=ceil(l/4), K=6, k=8,
               rotation keys X->X^5 and X->X^-1 generated at each level.
* ``n17``      N=2^17, L=40, dnum=5 (alpha=8), K=8, k=8, relinearise then
               rotate by X->X^5.
* ``bsgs16``   N=2^16, L=24, dnum=4, K=6, one ciphertext through a
               baby-step/giant-step linear transform of n1 x n2 = 4 x 4
               diagonals: baby rotations X->X^(5^i), i=1..3, giant rotations
               X->X^(5^(4j)), j=1..3, diagonals uniform over the extended basis.

Secrets are ternary with Hamming weight h (64 for ``tiny``, 192 otherwise);
errors are rounded Gaussians with sigma=3.2, tail-cut at |e| <= 19.  This
follows the Perseus README ('What's inside': keys regenerated from a ChaCha12
seed) for the seed-derived half and the usual RNS-CKKS key-generation recipe
for the rest.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SIGMA = 3.2
E_TAIL = 19

# numpy.random.default_rng([workload_index, stream, idx]) stream ids
STREAM_CT = 1
STREAM_SECRET = 2
STREAM_ERROR = 3
STREAM_KEY_B = 4  # uniform stand-in for a key's b half (benchmark only)
STREAM_PLAIN = 5  # plaintext diagonals of a linear transform


@dataclass(frozen=True)
class Workload:
    name: str
    index: int          # seed namespace for this workload
    log2n: int
    L: int              # q-primes at the top level
    dnum: int
    K: int              # special primes
    h: int              # Hamming weight of the ternary secret
    batch: tuple = (1,)
    levels: tuple = ()
    galois: tuple = ()  # Galois elements of the rotation keys (1 = relinearisation)
    hoisted: bool = False
    chain: bool = False  # relinearise then rotate
    extra: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        return 1 << self.log2n

    def level_list(self):
        return self.levels if self.levels else (self.L,)


def galois_rot(step: int, N: int) -> int:
    """Galois element of the rotation X -> X^(5^step) (mod 2N)."""
    return pow(5, step, 2 * N)


def galois_conj(N: int) -> int:
    """Galois element of X -> X^-1."""
    return 2 * N - 1


WORKLOADS = {
    "tiny": Workload("tiny", 0, 12, 3, 3, 1, 64, batch=(1,), galois=(5,)),
    "n16": Workload("n16", 1, 16, 24, 4, 6, 192, batch=(1, 8), galois=(1,)),
    "hoist16": Workload("hoist16", 2, 16, 24, 4, 6, 192, batch=(1,),
                        galois=tuple(galois_rot(r, 1 << 16) for r in range(1, 17)), hoisted=True),
    "levels16": Workload("levels16", 3, 16, 24, 4, 6, 192, batch=(8,), levels=(24, 20, 16, 12, 8, 4),
                         galois=(5, galois_conj(1 << 16))),
    "n17": Workload("n17", 4, 17, 40, 5, 8, 192, batch=(8,), galois=(1, 5), chain=True),
    "bsgs16": Workload("bsgs16", 5, 16, 24, 4, 6, 192, batch=(1,),
                       galois=tuple(galois_rot(r, 1 << 16) for r in (1, 2, 3, 4, 8, 12)),
                       extra={"n1": 4, "n2": 4}),
}


def rng(workload_index: int, stream: int, idx: int) -> np.random.Generator:
    return np.random.default_rng([workload_index, stream, idx])


def key_seed(workload_index: int, key_index: int) -> bytes:
    """32-byte ChaCha key of key number ``key_index``: LE32(workload) || LE32(key) || 24 zero bytes."""
    return (int(workload_index).to_bytes(4, "little") + int(key_index).to_bytes(4, "little") + bytes(24))


def uniform_limbs(g: np.random.Generator, moduli, N: int) -> np.ndarray:
    """[len(moduli)][N] uint32, limb j uniform in [0, moduli[j])."""
    out = np.empty((len(moduli), N), dtype=np.uint32)
    for j, m in enumerate(moduli):
        out[j] = g.integers(0, int(m), N, dtype=np.uint64).astype(np.uint32)
    return out


def ciphertexts(workload_index: int, q_primes, N: int, count: int, first: int = 0) -> np.ndarray:
    """[count][2][l][N] uint32 ciphertexts with every stored word uniform mod q_i.

    Ciphertext ``idx`` draws from stream (workload, 1, idx), limb by limb, c0 then c1.
    """
    q_primes = list(q_primes)
    out = np.empty((count, 2, len(q_primes), N), dtype=np.uint32)
    for c in range(count):
        g = rng(workload_index, STREAM_CT, first + c)
        out[c, 0] = uniform_limbs(g, q_primes, N)
        out[c, 1] = uniform_limbs(g, q_primes, N)
    return out


def ternary_secret(workload_index: int, N: int, h: int, idx: int = 0) -> np.ndarray:
    """int64 coefficients in {-1,0,1} with exactly h non-zeros at distinct positions."""
    g = rng(workload_index, STREAM_SECRET, idx)
    s = np.zeros(N, dtype=np.int64)
    pos = g.choice(N, size=h, replace=False)
    s[pos] = g.choice(np.array([-1, 1], dtype=np.int64), size=h)
    return s


def gaussian_errors(workload_index: int, key_index: int, count: int, N: int) -> np.ndarray:
    """[count][N] int64 rounded Gaussian (sigma 3.2), |e| <= 19 (redrawn beyond)."""
    g = rng(workload_index, STREAM_ERROR, key_index)
    out = np.empty((count, N), dtype=np.int64)
    for i in range(count):
        e = np.rint(g.normal(0.0, SIGMA, N)).astype(np.int64)
        bad = np.abs(e) > E_TAIL
        while bad.any():
            e[bad] = np.rint(g.normal(0.0, SIGMA, int(bad.sum()))).astype(np.int64)
            bad = np.abs(e) > E_TAIL
        out[i] = e
    return out


def uniform_key_b(workload_index: int, key_index: int, digits: int, moduli, N: int) -> np.ndarray:
    """[digits][len(moduli)][N] uint32 uniform words standing in for a key's b half.

    A real b half is computationally indistinguishable from uniform, so timing
    runs that must not depend on key generation use this draw.
    """
    g = rng(workload_index, STREAM_KEY_B, key_index)
    out = np.empty((digits, len(moduli), N), dtype=np.uint32)
    for d in range(digits):
        out[d] = uniform_limbs(g, moduli, N)
    return out


def small_plaintexts(workload_index: int, count: int, N: int, bound: int, idx: int = 0) -> np.ndarray:
    """[count][N] int64 coefficients uniform in [-bound, bound] (small plaintext polynomials)."""
    g = rng(workload_index, STREAM_PLAIN, idx)
    return g.integers(-bound, bound + 1, (count, N), dtype=np.int64)


def uniform_diagonals(workload_index: int, n2: int, n1: int, moduli, N: int) -> np.ndarray:
    """[n2][n1][len(moduli)][N] uint32 uniform words standing in for plaintext diagonals."""
    g = rng(workload_index, STREAM_PLAIN, 1000)
    out = np.empty((n2, n1, len(moduli), N), dtype=np.uint32)
    for j in range(n2):
        for i in range(n1):
            out[j, i] = uniform_limbs(g, moduli, N)
    return out
