"""Property tests of the oracle over random small shapes (CPU only, hypothesis).

The fixed-shape pins elsewhere check the oracle at the workloads' sizes; these
draw the ring degree, the prime, the digit partition and the inputs at random
and check the same definitions and invariants:

* the NTT: the inverse undoes it, it turns the negacyclic schoolbook product
  into a pointwise one, and entry j is a(psi^(2j+1)) evaluated with Python ints;
* automorphisms compose as X -> X^(k k') and the conjugation is an involution;
* ModUp: for every digit the converted limbs hold S mod t for the integer
  S = sum_i y_i (Q_d/q_i), and S - CRT(c1 on D_d) = u Q_d with 0 <= u < alpha_d;
* ModDown: out P + C = acc over Q P with C = [acc]_P + v P, 0 <= v < K.
"""

import math

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import keyswitch as ks
from oracle import rns

U64 = np.uint64
SETTINGS = settings(max_examples=20, deadline=None, suppress_health_check=[HealthCheck.too_slow])


def _crt(residues, moduli):
    M = math.prod(moduli)
    x = 0
    for r, m in zip(residues, moduli):
        Mi = M // m
        x += int(r) * Mi * pow(Mi % m, -1, m)
    return x % M


@SETTINGS
@given(log2n=st.integers(3, 8), pick=st.integers(0, 15), seed=st.integers(0, 2**32 - 1))
def test_ntt_definition_roundtrip_and_convolution(log2n, pick, seed):
    N = 1 << log2n
    q = rns.ntt_primes(N, 16)[pick]
    psi = rns.find_psi(q, N)
    g = np.random.default_rng(seed)
    a = g.integers(0, q, N, dtype=np.uint64)
    b = g.integers(0, q, N, dtype=np.uint64)
    ah = rns.ntt(a, q)
    assert np.array_equal(rns.intt(ah, q), a)
    for j in g.integers(0, N, 3):
        x = pow(psi, 2 * int(j) + 1, q)
        assert int(ah[j]) == sum(int(a[i]) * pow(x, i, q) for i in range(N)) % q
    prod = [0] * N
    for i in range(N):
        for k in range(N):
            v = int(a[i]) * int(b[k])
            if i + k < N:
                prod[i + k] += v
            else:
                prod[i + k - N] -= v
    want = np.array([v % q for v in prod], dtype=np.uint64)
    assert np.array_equal(rns.intt(ah * rns.ntt(b, q) % U64(q), q), want)


@SETTINGS
@given(log2n=st.integers(3, 9), k1=st.integers(0, 2**20), k2=st.integers(0, 2**20), seed=st.integers(0, 2**32 - 1))
def test_automorphisms_compose(log2n, k1, k2, seed):
    N = 1 << log2n
    g1, g2 = (2 * k1 + 1) % (2 * N), (2 * k2 + 1) % (2 * N)
    x = np.random.default_rng(seed).integers(0, 1 << 31, N, dtype=np.uint64)
    assert np.array_equal(ks.automorphism(ks.automorphism(x, g1), g2), ks.automorphism(x, g1 * g2 % (2 * N)))
    conj = 2 * N - 1
    assert np.array_equal(ks.automorphism(ks.automorphism(x, conj), conj), x)


@st.composite
def shapes(draw):
    L = draw(st.integers(1, 6))
    dnum = draw(st.integers(1, L))
    K = draw(st.integers(1, 3))
    level = draw(st.integers(1, L))
    partition = draw(st.integers(0, 1))
    return L, dnum, K, level, partition


@SETTINGS
@given(shape=shapes(), seed=st.integers(0, 2**32 - 1))
def test_modup_conversion_invariant(shape, seed):
    L, dnum, K, level, partition = shape
    prm = ks.Params(4, L, dnum, K, partition=partition)
    g = np.random.default_rng(seed)
    c1 = np.stack([g.integers(0, q, prm.N, dtype=np.uint64) for q in prm.q[:level]])
    ext = ks.modup(prm, c1, level)
    basis = prm.basis(level)
    coef = [rns.intt(c1[i], prm.q[i]) for i in range(level)]
    for d, D in enumerate(prm.digits(level)):
        Qd = math.prod(prm.q[i] for i in D)
        ext_coef = [rns.intt(ext[d, t], r) for t, r in enumerate(basis)]
        for n in range(prm.N):
            y = {i: int(coef[i][n]) * pow((Qd // prm.q[i]) % prm.q[i], -1, prm.q[i]) % prm.q[i] for i in D}
            S = sum(y[i] * (Qd // prm.q[i]) for i in D)
            x = _crt([int(coef[i][n]) for i in D], [prm.q[i] for i in D])
            assert (S - x) % Qd == 0 and 0 <= (S - x) // Qd < len(D)
            for t, r in enumerate(basis):
                if t in D:
                    continue
                assert int(ext_coef[t][n]) == S % r


@SETTINGS
@given(shape=shapes(), seed=st.integers(0, 2**32 - 1))
def test_moddown_floor_invariant(shape, seed):
    L, dnum, K, level, partition = shape
    prm = ks.Params(4, L, dnum, K, partition=partition)
    basis = prm.basis(level)
    g = np.random.default_rng(seed)
    acc = np.stack([g.integers(0, r, prm.N, dtype=np.uint64) for r in basis])
    out = ks.moddown(prm, acc, level)
    P, Q = prm.P, math.prod(prm.q[:level])
    acc_coef = [rns.intt(acc[t], r) for t, r in enumerate(basis)]
    out_coef = [rns.intt(out[i], prm.q[i]) for i in range(level)]
    for n in range(prm.N):
        A = _crt([int(acc_coef[t][n]) for t in range(len(basis))], basis)
        o = _crt([int(out_coef[i][n]) for i in range(level)], list(prm.q[:level]))
        C = (A - o * P) % (Q * P)
        assert C % P == A % P and C // P < K
