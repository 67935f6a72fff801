"""The C++ oracle tier (oracle/ks_o2.cpp) against the pages' mathematics and the numpy oracle (CPU).

Pins of its own, independent of the numpy oracle: primes and roots checked
by their definitions, the NTT by direct evaluation a_hat[j] = a(psi^(2j+1))
with Python integers and by the negacyclic convolution theorem against a
schoolbook product, ChaCha20 against the OpenSSL command line and the zero-round
state layout. Then the two oracles, written apart and sharing no code, agree
word for word: on random small shapes (both partitions, ragged digits,
automorphisms, stored and regenerated key halves) and at the full sizes,
where the C++ tier re-derives digests the numpy oracle stored.
"""

import os
import random
import shutil
import subprocess
import sys

import numpy as np
import pytest

from oracle import chacha, o2
from oracle import keyswitch as ks
from oracle import rns

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden"))
import cases  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _built():
    o2.lib()


# ---------------------------------------------------------------------------
# pins of the C++ tier by definition
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("log2n", [6, 10, 12, 16, 17])
def test_primes_are_the_largest_ntt_friendly_primes(log2n):
    """Every prime = 1 mod 2N below 2^31, largest first, none skipped (each candidate in the
    range tested by deterministic Miller-Rabin, which the RNS tests pin)."""
    O = o2.O2(log2n, 6, 3, 3)
    N = 1 << log2n
    pr, psi = O.tables()
    assert pr == sorted(pr, reverse=True) and pr[0] < 1 << 31
    for p in pr:
        assert p % (2 * N) == 1 and rns.is_prime(p)
    # nothing of the form 1 mod 2N was skipped between 2^31 and the last prime
    for c in range(pr[-1], 1 << 31, 2 * N):
        assert (c in pr) == rns.is_prime(c)
    for p, w in zip(pr, psi):
        assert pow(w, N, p) == p - 1


@pytest.mark.parametrize("log2n", [12, 14, 16])
def test_psi_is_the_smallest_root(log2n):
    """psi is the smallest x >= 2 with x^N = -1: no smaller x qualifies (brute force; about
    2^31/N candidates, so the sizes stay at N >= 2^12)."""
    O = o2.O2(log2n, 2, 1, 1)
    N = 1 << log2n
    for p, w in zip(*O.tables()):
        assert pow(w, N, p) == p - 1
        assert all(pow(x, N, p) != p - 1 for x in range(2, w))


def test_ntt_is_direct_evaluation_small():
    """N = 64, every output: a_hat[j] = sum_i a_i psi^((2j+1) i) with Python integers."""
    O = o2.O2(6, 3, 1, 2)
    N = 64
    rng = random.Random(1)
    for k, (p, w) in enumerate(zip(*O.tables())):
        a = [rng.randrange(p) for _ in range(N)]
        got = O.ntt(a, k)
        for j in range(N):
            x = pow(w, 2 * j + 1, p)
            assert int(got[j]) == sum(ai * pow(x, i, p) for i, ai in enumerate(a)) % p
        assert O.ntt(got, k, inverse=True).tolist() == a


@pytest.mark.parametrize("log2n", [12, 16, 17])
def test_ntt_direct_evaluation_sampled(log2n):
    """Full-size transforms: 12 sampled outputs by Horner's rule at psi^(2j+1); round trip exact."""
    O = o2.O2(log2n, 2, 1, 1)
    N = 1 << log2n
    rng = np.random.default_rng(log2n)
    for k, (p, w) in enumerate(zip(*O.tables())):
        a = rng.integers(0, p, N, dtype=np.uint64)
        got = O.ntt(a, k)
        coeffs = [int(v) for v in a[::-1]]
        for j in rng.integers(0, N, 12):
            x = pow(w, 2 * int(j) + 1, p)
            acc = 0
            for cf in coeffs:
                acc = (acc * x + cf) % p
            assert int(got[j]) == acc
        assert np.array_equal(O.ntt(got, k, inverse=True), a.astype(np.uint32))


def test_ntt_convolution_theorem():
    """NTT(a) * NTT(b) = NTT(a b mod X^N + 1) with the product taken by schoolbook."""
    O = o2.O2(7, 2, 1, 1)
    N = 128
    rng = random.Random(7)
    for k, p in enumerate(O.tables()[0]):
        a = [rng.randrange(p) for _ in range(N)]
        b = [rng.randrange(p) for _ in range(N)]
        c = [0] * N
        for i in range(N):
            for j in range(N):
                if i + j < N:
                    c[i + j] += a[i] * b[j]
                else:
                    c[i + j - N] -= a[i] * b[j]
        c = [x % p for x in c]
        prod = O.ntt(a, k).astype(np.uint64) * O.ntt(b, k).astype(np.uint64) % np.uint64(p)
        assert prod.tolist() == O.ntt(c, k).tolist()


def test_ntt_matches_the_numpy_oracle():
    O = o2.O2(12, 3, 1, 2)
    rng = np.random.default_rng(3)
    for k, p in enumerate(O.tables()[0]):
        a = rng.integers(0, p, O.N, dtype=np.uint64)
        assert np.array_equal(O.ntt(a, k).astype(np.uint64), rns.ntt(a, p))
        assert np.array_equal(O.ntt(a, k, inverse=True).astype(np.uint64), rns.intt(a, p))


HAVE_OPENSSL = shutil.which("openssl") is not None


@pytest.mark.skipif(not HAVE_OPENSSL, reason="openssl command line not available")
@pytest.mark.parametrize("case", range(4))
def test_chacha20_matches_openssl(case):
    rnd = random.Random(100 + case)
    key = bytes(rnd.randrange(256) for _ in range(32))
    nonce = (0, rnd.randrange(8), rnd.randrange(64)) if case % 2 else tuple(rnd.randrange(1 << 32) for _ in range(3))
    counter = 0 if case < 2 else rnd.randrange(1 << 20)
    iv = counter.to_bytes(4, "little") + b"".join(int(w).to_bytes(4, "little") for w in nonce)
    ref = subprocess.run(["openssl", "enc", "-chacha20", "-K", key.hex(), "-iv", iv.hex()], input=bytes(64 * 4),
                         stdout=subprocess.PIPE, check=True).stdout
    got = o2.chacha_blocks(key, counter, nonce, 4, rounds=20)
    assert got.tobytes() == ref


def test_chacha_zero_rounds_is_twice_the_state():
    key = bytes(range(50, 82))
    out = o2.chacha_blocks(key, 9, (1, 2, 3), 2, rounds=0)
    kw = [int.from_bytes(key[4 * i: 4 * i + 4], "little") for i in range(8)]
    for b in range(2):
        state = [0x61707865, 0x3320646E, 0x79622D32, 0x6B206574] + kw + [9 + b, 1, 2, 3]
        assert out[b].tolist() == [(2 * s) % (1 << 32) for s in state]


@pytest.mark.parametrize("rounds", [12, 20])
def test_chacha_matches_the_numpy_oracle(rounds):
    key = bytes(range(7, 39))
    got = o2.chacha_blocks(key, 5, (0, 3, 11), 6, rounds=rounds)
    assert np.array_equal(got, chacha.chacha_blocks(key, (0, 3, 11), np.arange(5, 11, dtype=np.uint32), rounds))


def test_bad_arguments_are_rejected():
    with pytest.raises(ValueError):
        o2.O2(3, 4, 2, 1)
    with pytest.raises(ValueError):
        o2.O2(10, 4, 5, 1)  # dnum > L
    O = o2.O2(10, 4, 2, 1)
    N = O.N
    ct = np.zeros((2, 4, N), dtype=np.uint32)
    b = np.zeros((2, 5, N), dtype=np.uint32)
    with pytest.raises(ValueError):
        O.keyswitch(ct, 4, 2, b, seed=bytes(32))  # even Galois element
    with pytest.raises(ValueError):
        O.keyswitch(ct, 4, 1, b)  # neither seed nor stored half
    bad = ct.copy()
    bad[0, 0, 0] = O.primes[0]
    with pytest.raises(ValueError):
        O.keyswitch(bad, 4, 1, b, seed=bytes(32))  # non-canonical word


# ---------------------------------------------------------------------------
# the two oracles agree
# ---------------------------------------------------------------------------

def _uniform(rng, moduli, N, lead=()):
    return np.stack([rng.integers(0, r, lead + (N,), dtype=np.uint64) for r in moduli], axis=len(lead))


# (log2n, L, dnum, K, partition, level, galois selector, stored a)
SHAPES = [
    (10, 6, 3, 2, 0, 6, "relin", False),
    (10, 6, 3, 2, 0, 5, "rot", False),      # ragged last digit
    (10, 7, 2, 3, 1, 7, "conj", True),
    (11, 7, 2, 3, 1, 3, "rot", False),      # partition 1 below the top: one digit, unused key limbs
    (10, 5, 5, 1, 0, 5, "rot", False),      # alpha = 1, K = 1
    (10, 4, 1, 4, 0, 4, "relin", True),     # one digit
    (11, 9, 3, 4, 0, 8, "rot", True),
    (10, 16, 2, 8, 0, 16, "conj", False),   # alpha = 8, K = 8
    (12, 8, 4, 2, 1, 5, "rot", False),
    (10, 12, 4, 3, 0, 1, "relin", False),   # level 1
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_keyswitch_agrees_with_the_numpy_oracle(shape):
    log2n, L, dnum, K, part, level, gsel, stored = shape
    prm = ks.Params(log2n, L, dnum, K, partition=part)
    O = o2.O2(log2n, L, dnum, K, partition=part)
    assert tuple(O.primes) == prm.primes
    N = prm.N
    rng = np.random.default_rng(1000 + SHAPES.index(shape))
    galois = {"relin": 1, "conj": 2 * N - 1, "rot": pow(5, int(rng.integers(1, N // 2)), 2 * N)}[gsel]
    kl = prm.key_level(level)
    beta_key = len(prm.digits(kl))
    basis = prm.basis(kl)
    b = _uniform(rng, basis, N, (beta_key,))
    a = _uniform(rng, basis, N, (beta_key,)) if stored else None
    seed = bytes(rng.integers(0, 256, 32, dtype=np.uint8))
    key = ks.Key(b=b, seed=seed, level=kl, galois=galois, a=a)
    ct = _uniform(rng, prm.q[:level], N, (2,))
    want = ks.keyswitch(prm, ct, key, level)
    got = O.keyswitch(ct, level, galois, b, seed=seed, evk_a=a)
    assert np.array_equal(got.astype(np.uint64), want)


def test_extreme_words_agree():
    """All-zero and all-(q-1) ciphertexts, b = r - 1 everywhere, at N = 2^11."""
    prm = ks.Params(11, 6, 2, 3)
    O = o2.O2(11, 6, 2, 3)
    N, level = prm.N, 6
    basis = prm.basis(level)
    beta = len(prm.digits(level))
    b = np.broadcast_to(np.array(basis, dtype=np.uint64)[None, :, None] - 1, (beta, len(basis), N)).copy()
    q = np.array(prm.q, dtype=np.uint64)[:, None]
    for ct in (np.zeros((2, level, N), dtype=np.uint64), np.broadcast_to(q - 1, (2, level, N)).copy()):
        key = ks.Key(b=b, seed=bytes(range(32)), level=level, galois=2 * N - 1)
        want = ks.keyswitch(prm, ct, key, level)
        assert np.array_equal(O.keyswitch(ct, level, 2 * N - 1, b, seed=bytes(range(32))).astype(np.uint64), want)


# ---------------------------------------------------------------------------
# full sizes: the C++ tier re-derives the stored digests
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def doc():
    return cases.load_digests()


def _o2_for(c):
    return o2.O2(c.prm.log2n, c.prm.L, c.prm.dnum, c.prm.K, c.prm.partition)


def _items(c, keys_items):
    """Digests of the C++ tier for (key index, ciphertext index) pairs of case c."""
    O = _o2_for(c)
    out = {}
    for r, bi in keys_items:
        k = c.keys[r]
        y = O.keyswitch(c.cts[bi], c.level, k.galois, k.b, seed=k.seed, evk_a=k.a)
        out[r * c.batch + bi] = cases.digest(y)
    return out


def test_fullsize_relinearisation_digests(doc):
    """N=2^16, L=24, dnum=4, K=6 under the workload's generated relinearisation key."""
    c = cases.case_n16_relin_k8()
    got = _items(c, [(0, 0), (0, 7)])
    want = doc["cases"]["n16_relin_k8"]["digests"]
    assert all(want[i] == d for i, d in got.items())


def test_fullsize_extreme_digests(doc):
    """All-zero, all-(q-1) and maximal-ModUp ciphertexts under both extreme keys."""
    cx, cy = cases.case_n16_extreme()
    for c in (cx, cy):
        got = _items(c, [(0, 0), (0, 1), (0, 2)])
        want = doc["cases"][c.name]["digests"]
        assert all(want[i] == d for i, d in got.items()), c.name


def test_fullsize_level_and_hoist_digests(doc):
    c = cases.case_n16_level(4)
    got = _items(c, [(0, 3), (1, 3)])
    assert all(doc["cases"]["n16_level4"]["digests"][i] == d for i, d in got.items())
    c = cases.case_n16_hoist16()
    got = _items(c, [(5, 0), (15, 0)])
    assert all(doc["cases"]["n16_hoist16"]["digests"][i] == d for i, d in got.items())


def test_fullsize_n17_chain_digests(doc):
    """N=2^17, L=40, dnum=5, K=8: item 0 relinearised, then rotated by X -> X^5."""
    c = cases.case_n17_chain()
    O = _o2_for(c)
    relin, rot = c.keys
    step1 = O.keyswitch(c.cts[0], c.level, relin.galois, relin.b, seed=relin.seed)
    step2 = O.keyswitch(step1, c.level, rot.galois, rot.b, seed=rot.seed)
    want = doc["cases"]["n17_chain"]["digests"]
    assert cases.digest(step1) == want[0]
    assert cases.digest(step2) == want[8]
