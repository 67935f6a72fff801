"""Primes, roots and the negacyclic NTT (oracle; test infrastructure only).

Readings of the pages (which name NTT kernels over a 32-bit prime chain but
give no formulas; Perseus README, 'Layout' and the opening paragraph on the
32-bit FIDESlib port):

* primes: every prime q < 2^31 with q = 1 (mod 2N), taken in descending
  order; the first L are the ciphertext primes q_0..q_{L-1}, the next K the
  special primes p_0..p_{K-1}.
* psi: the smallest integer x >= 2 with x^N = -1 (mod q), i.e. the smallest
  primitive 2N-th root of unity.
* evaluation layout: natural order, a_hat[j] = a(psi^(2j+1)) mod q.
"""

from __future__ import annotations

from functools import lru_cache

import numpy as np

_MR_BASES = (2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37)


def is_prime(n: int) -> bool:
    """Deterministic Miller-Rabin (the bases above are exact for n < 3.3e24)."""
    if n < 2:
        return False
    for p in _MR_BASES:
        if n % p == 0:
            return n == p
    d, s = n - 1, 0
    while d % 2 == 0:
        d //= 2
        s += 1
    for a in _MR_BASES:
        x = pow(a, d, n)
        if x in (1, n - 1):
            continue
        for _ in range(s - 1):
            x = x * x % n
            if x == n - 1:
                break
        else:
            return False
    return True


def ntt_primes(N: int, count: int, below: int = 1 << 31) -> list[int]:
    """The ``count`` largest primes q < ``below`` with q = 1 (mod 2N), descending."""
    m = 2 * N
    q = ((below - 2) // m) * m + 1
    out = []
    while len(out) < count:
        if q < 2:
            raise ValueError("not enough NTT-friendly primes")
        if is_prime(q):
            out.append(q)
        q -= m
    return out


@lru_cache(maxsize=None)
def find_psi(q: int, N: int) -> int:
    """Smallest primitive 2N-th root of unity mod q (N a power of two).

    The primitive 2N-th roots are exactly the odd powers r0^t (t odd, t < 2N)
    of any one of them, r0 = g^((q-1)/2N) for a generator-like g; take the
    minimum over that set.
    """
    assert (q - 1) % (2 * N) == 0
    for g in range(2, q):
        r0 = pow(g, (q - 1) // (2 * N), q)
        if pow(r0, N, q) == q - 1:
            break
    best = r0
    r2 = r0 * r0 % q
    x = r0
    for _ in range(N - 1):
        x = x * r2 % q
        if x < best:
            best = x
    return best


@lru_cache(maxsize=None)
def _powers(base: int, n: int, q: int) -> np.ndarray:
    """[base^0, base^1, ..., base^(n-1)] mod q as uint64."""
    out = np.empty(n, dtype=np.uint64)
    x = 1
    for i in range(n):
        out[i] = x
        x = x * base % q
    out.setflags(write=False)
    return out


@lru_cache(maxsize=None)
def _bitrev(N: int) -> np.ndarray:
    bits = N.bit_length() - 1
    idx = np.arange(N, dtype=np.int64)
    rev = np.zeros(N, dtype=np.int64)
    for b in range(bits):
        rev |= ((idx >> b) & 1) << (bits - 1 - b)
    rev.setflags(write=False)
    return rev


def _cyclic_dft(x: np.ndarray, omega: int, q: int) -> np.ndarray:
    """X[j] = sum_i x[i] * omega^(i*j) mod q (length N, omega of order N).

    Textbook iterative radix-2 decimation-in-time FFT: permute the input to
    bit-reversed order, then merge transforms of size m into size 2m with
    X[k] = E[k] + w^k O[k], X[k+m] = E[k] - w^k O[k].
    """
    N = x.shape[-1]
    x = x[_bitrev(N)].astype(np.uint64)
    m = 1
    while m < N:
        w = _powers(pow(omega, N // (2 * m), q), m, q)
        x = x.reshape(N // (2 * m), 2, m)
        even = x[:, 0, :]
        odd = x[:, 1, :] * w % q
        x = np.stack(((even + odd) % q, (even + (q - odd)) % q), axis=1).reshape(N)
        m *= 2
    return x


def ntt(a: np.ndarray, q: int) -> np.ndarray:
    """Negacyclic NTT of one limb: a_hat[j] = sum_i a[i] psi^((2j+1) i) mod q.

    Computed as a pre-twist by psi^i followed by a cyclic DFT with
    omega = psi^2 (psi^((2j+1)i) = psi^i * omega^(ij)).
    """
    a = np.asarray(a, dtype=np.uint64)
    N = a.shape[-1]
    psi = find_psi(q, N)
    return _cyclic_dft(a * _powers(psi, N, q) % q, psi * psi % q, q)


def intt(a_hat: np.ndarray, q: int) -> np.ndarray:
    """Inverse of :func:`ntt`: a[i] = N^-1 psi^-i sum_j a_hat[j] omega^(-ij) mod q."""
    a_hat = np.asarray(a_hat, dtype=np.uint64)
    N = a_hat.shape[-1]
    psi = find_psi(q, N)
    psi_inv = pow(psi, -1, q)
    x = _cyclic_dft(a_hat, psi_inv * psi_inv % q, q)
    n_inv = pow(N, -1, q)
    return x * _powers(psi_inv, N, q) % q * n_inv % q


def to_residues(coeffs: np.ndarray, q: int) -> np.ndarray:
    """Signed integer coefficients -> canonical residues mod q (uint64)."""
    return (np.asarray(coeffs, dtype=np.int64) % q).astype(np.uint64)


def centered(x: np.ndarray, q: int) -> np.ndarray:
    """Canonical residues -> representatives in (-q/2, q/2] as int64."""
    x = np.asarray(x, dtype=np.int64)
    return np.where(x > q // 2, x - q, x)
