"""Pins of the oracle's primes, roots, NTT and automorphism (CPU only).

Each check compares the oracle with something other than itself: sympy's
primality test, brute-force searches, the NTT's defining sum evaluated with
Python integers, the negacyclic convolution theorem with a schoolbook
product, Horner evaluation at full size, and the coefficient-domain
definition of X -> X^k.
"""

import random

import numpy as np
import pytest
import sympy

from oracle import keyswitch as ks
from oracle import rns


@pytest.mark.parametrize("log2n,count", [(12, 4), (16, 30), (17, 48)])
def test_prime_rule(log2n, count):
    N = 1 << log2n
    ps = rns.ntt_primes(N, count)
    assert ps == sorted(ps, reverse=True)
    for p in ps:
        assert p < (1 << 31) and p % (2 * N) == 1 and sympy.isprime(p)
    # nothing skipped: every candidate = 1 mod 2N between the chosen ones is composite
    top = ((1 << 31) - 2) // (2 * N) * (2 * N) + 1
    chosen = set(ps)
    for c in range(top, ps[-1] - 1, -2 * N):
        assert (c in chosen) == bool(sympy.isprime(c)), c


def test_prime_values_small_ring():
    # N = 2^12: the three ciphertext primes and the special prime, descending
    assert rns.ntt_primes(1 << 12, 4) == [2147377153, 2147352577, 2147295233, 2147205121]


def test_is_prime_against_sympy():
    rnd = random.Random(1)
    for _ in range(3000):
        n = rnd.randrange(2, 1 << 40)
        assert rns.is_prime(n) == bool(sympy.isprime(n))
    for n in (2, 3, 4, 561, 1105, 2147483647, 2147483649, 3215031751):
        assert rns.is_prime(n) == bool(sympy.isprime(n))


@pytest.mark.parametrize("q,N", [(17, 8), (97, 16), (193, 32), (257, 64), (7681, 256), (12289, 512)])
def test_psi_is_smallest_root_small(q, N):
    psi = rns.find_psi(q, N)
    roots = [x for x in range(2, q) if pow(x, N, q) == q - 1]
    assert psi == min(roots)


@pytest.mark.parametrize("log2n,which", [(12, 0), (16, 0), (16, 5), (17, 0)])
def test_psi_is_smallest_root_real(log2n, which):
    N = 1 << log2n
    q = rns.ntt_primes(N, which + 1)[which]
    psi = rns.find_psi(q, N)
    assert pow(psi, N, q) == q - 1
    for x in range(2, psi):
        assert pow(x, N, q) != q - 1


def _dft_definition(a, q, psi):
    N = len(a)
    return [sum(int(a[i]) * pow(psi, (2 * j + 1) * i, q) for i in range(N)) % q for j in range(N)]


@pytest.mark.parametrize("N", [2, 8, 16, 64])
def test_ntt_matches_definition(N):
    rnd = np.random.default_rng(N)
    for q in (rns.ntt_primes(1 << 12, 2) + [257 if N <= 128 else 12289]):
        if (q - 1) % (2 * N):
            continue
        a = rnd.integers(0, q, N, dtype=np.uint64)
        psi = rns.find_psi(q, N)
        assert rns.ntt(a, q).tolist() == _dft_definition(a.tolist(), q, psi)


def _schoolbook_negacyclic(a, b, q):
    N = len(a)
    out = [0] * N
    for i in range(N):
        for j in range(N):
            k = i + j
            if k < N:
                out[k] += int(a[i]) * int(b[j])
            else:
                out[k - N] -= int(a[i]) * int(b[j])
    return [x % q for x in out]


@pytest.mark.parametrize("N", [32, 256])
def test_ntt_convolution_theorem(N):
    q = rns.ntt_primes(1 << 12, 1)[0]
    rnd = np.random.default_rng(7)
    a = rnd.integers(0, q, N, dtype=np.uint64)
    b = rnd.integers(0, q, N, dtype=np.uint64)
    prod = np.array(_schoolbook_negacyclic(a, b, q), dtype=np.uint64)
    lhs = rns.ntt(a, q) * rns.ntt(b, q) % np.uint64(q)
    assert np.array_equal(lhs, rns.ntt(prod, q))


@pytest.mark.parametrize("log2n", [4, 12, 16])
def test_intt_inverts_ntt(log2n):
    N = 1 << log2n
    for q in rns.ntt_primes(N, 2):
        x = np.random.default_rng(q).integers(0, q, N, dtype=np.uint64)
        assert np.array_equal(rns.intt(rns.ntt(x, q), q), x)
        assert np.array_equal(rns.ntt(rns.intt(x, q), q), x)


@pytest.mark.parametrize("log2n", [16, 17])
def test_ntt_full_size_horner(log2n):
    """Spot values of the full-size NTT equal a(psi^(2j+1)) by Horner's rule."""
    N = 1 << log2n
    q = rns.ntt_primes(N, 3)[2]
    a = np.random.default_rng(log2n).integers(0, q, N, dtype=np.uint64)
    ah = rns.ntt(a, q)
    psi = rns.find_psi(q, N)
    coeffs = [int(v) for v in a[::-1]]
    for j in (0, 1, N // 3, N - 1):
        x = pow(psi, 2 * j + 1, q)
        acc = 0
        for c in coeffs:
            acc = (acc * x + c) % q
        assert int(ah[j]) == acc


def _automorphism_coeff(a, k, q):
    """a(X^k) mod (X^N + 1): coefficient i moves to i*k mod 2N, negated past N."""
    N = len(a)
    out = [0] * N
    for i in range(N):
        e = i * k % (2 * N)
        if e < N:
            out[e] = (out[e] + int(a[i])) % q
        else:
            out[e - N] = (out[e - N] - int(a[i])) % q
    return np.array(out, dtype=np.uint64)


@pytest.mark.parametrize("k", [1, 3, 5, 25, 125, 127])
def test_automorphism_matches_coefficient_definition(k):
    N = 64
    q = rns.ntt_primes(1 << 12, 1)[0]
    a = np.random.default_rng(k).integers(0, q, N, dtype=np.uint64)
    lhs = rns.ntt(_automorphism_coeff(a, k, q), q)
    rhs = ks.automorphism(rns.ntt(a, q), k)
    assert np.array_equal(lhs, rhs)


def test_automorphism_group_law():
    N = 1 << 10
    x = np.arange(N, dtype=np.uint64)
    for k1, k2 in [(5, 25), (2 * N - 1, 5), (3, 7)]:
        two = ks.automorphism(ks.automorphism(x, k1), k2)
        assert np.array_equal(two, ks.automorphism(x, k1 * k2 % (2 * N)))
    assert np.array_equal(ks.automorphism(ks.automorphism(x, 2 * N - 1), 2 * N - 1), x)
