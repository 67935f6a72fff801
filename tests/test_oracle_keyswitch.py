"""Pins of the oracle's ModUp, ModDown and whole key switch (CPU only).

ModUp and ModDown are checked coefficient by coefficient against exact CRT
reconstruction with big integers (sympy): fast base conversion must return
x + u*Q_d with 0 <= u < alpha_d (exactly x when alpha_d = 1), and ModDown's
output times P must equal acc - C with C = [acc]_P + v*P, 0 <= v < K. The
whole key switch is checked by decrypting under the real secrets: the error
must be the same small integer polynomial on every limb and stay within the
analytic bound. Planted mistakes in a copy of the oracle must fail the check.
"""

import math

import numpy as np
import pytest
from sympy.ntheory.modular import crt

import ks_inputs as ki
from oracle import keyswitch as ks
from oracle import rns


def small_params(log2n=6, L=6, dnum=3, K=2, rounds=12):
    return ks.Params(log2n, L, dnum, K, chacha_rounds=rounds)


def _coef(limbs, moduli):
    return [rns.intt(limbs[j], m) for j, m in enumerate(moduli)]


@pytest.mark.parametrize("L,dnum,level", [(6, 3, 6), (6, 2, 6), (5, 2, 5), (6, 3, 4), (3, 3, 3)])
def test_modup_is_fast_base_conversion(L, dnum, level):
    prm = small_params(L=L, dnum=dnum)
    N = prm.N
    c1 = ki.uniform_limbs(np.random.default_rng(L * 10 + level), prm.q[:level], N)
    ext = ks.modup(prm, c1, level)
    basis = prm.basis(level)
    c1_coef = _coef(c1, prm.q[:level])
    for d, D in enumerate(prm.digits(level)):
        Qd = math.prod(prm.q[i] for i in D)
        ext_coef = _coef(ext[d], basis)
        for i in D:  # the digit's own limbs are passed through
            assert np.array_equal(ext[d, i], c1[i])
        others = [j for j in range(len(basis)) if j not in D]
        for n in range(N):
            x = int(crt([prm.q[i] for i in D], [int(c1_coef[i][n]) for i in D])[0])
            us = set()
            for j in others:
                t = basis[j]
                z = int(ext_coef[j][n])
                # find u with z = x + u*Qd (mod t), 0 <= u < alpha
                cand = [u for u in range(len(D)) if (x + u * Qd - z) % t == 0]
                assert len(cand) == 1, (d, j, n)
                us.add(cand[0])
            assert len(us) == 1  # the same u on every target
            if len(D) == 1:
                assert us == {0}


@pytest.mark.parametrize("K,level", [(1, 3), (2, 6), (3, 5)])
def test_moddown_floor_invariant(K, level):
    prm = small_params(L=6, dnum=3, K=K)
    N = prm.N
    basis = prm.basis(level)
    acc = ki.uniform_limbs(np.random.default_rng(K), basis, N)
    out = ks.moddown(prm, acc, level)
    acc_coef = _coef(acc, basis)
    out_coef = _coef(out, prm.q[:level])
    P = prm.P
    Q = math.prod(prm.q[:level])
    for n in range(N):
        A = int(crt(basis, [int(acc_coef[j][n]) for j in range(len(basis))])[0])
        O = int(crt(list(prm.q[:level]), [int(out_coef[i][n]) for i in range(level)])[0])
        D = (A - P * O) % (P * Q)
        assert D % P == A % P and D < K * P


def _keys_and_secret(prm, widx, level, galois_list, h):
    s = ki.ternary_secret(widx, prm.N, h)
    keys, emax = [], 0
    for kidx, g in enumerate(galois_list):
        errs = ki.gaussian_errors(widx, kidx, len(prm.digits(level)), prm.N)
        emax = max(emax, int(np.abs(errs).max()))
        keys.append(ks.keygen(prm, s, errs, ki.key_seed(widx, kidx), level, g))
    return s, keys, emax


def _check_decrypts(prm, ct, out, s, galois, level, emax, h):
    e = ks.decryption_error(prm, ct, out, s, galois, level)
    assert e is not None, "error residues differ between limbs"
    B = ks.error_bound(prm, level, emax, h)
    assert np.abs(e).max() <= B
    return e


def test_tiny_rotation_decrypts():
    w = ki.WORKLOADS["tiny"]
    prm = ks.Params(w.log2n, w.L, w.dnum, w.K)
    s, (key,), emax = _keys_and_secret(prm, w.index, w.L, (5,), w.h)
    assert key.seed == bytes(32)
    ct = ki.ciphertexts(w.index, prm.q, prm.N, 1)[0]
    out = ks.keyswitch(prm, ct, key, w.L)
    e = _check_decrypts(prm, ct, out, s, 5, w.L, emax, w.h)
    assert np.abs(e).max() > 0  # a real, noisy key switch


@pytest.mark.parametrize("galois,level", [(1, 6), (5, 6), (127, 4), (25, 5), (1, 1)])
def test_small_keyswitch_decrypts(galois, level):
    prm = small_params(log2n=6, L=6, dnum=3, K=2)
    s, (key,), emax = _keys_and_secret(prm, 9, level, (galois,), 8)
    ct = ki.ciphertexts(9, prm.q[:level], prm.N, 1)[0]
    out = ks.keyswitch(prm, ct, key, level)
    _check_decrypts(prm, ct, out, s, galois, level, emax, 8)


def test_hoisted_equals_singles_and_stored_equals_regenerated():
    prm = small_params(log2n=7, L=4, dnum=2, K=2)
    level = 4
    s, keys, _ = _keys_and_secret(prm, 5, level, (5, 25, 255), 10)
    ct = ki.ciphertexts(5, prm.q, prm.N, 1)[0]
    hoisted = ks.keyswitch_hoisted(prm, ct, keys, level)
    for r, key in enumerate(keys):
        assert np.array_equal(hoisted[r], ks.keyswitch(prm, ct, key, level))
        stored = ks.Key(b=key.b, seed=None, level=level, galois=key.galois, a=ks.key_a(prm, key))
        assert np.array_equal(ks.keyswitch(prm, ct, stored, level), hoisted[r])


def test_top_level_partition_serves_every_level():
    """Partition 1: alpha = ceil(L/dnum) at every level and one key generated at
    level L; a ciphertext at any lower level key-switches within the bound."""
    prm = ks.Params(6, 7, 3, 3, partition=1)
    assert [prm.alpha(l) for l in (7, 5, 2)] == [3, 3, 3]
    assert prm.digits(5) == [[0, 1, 2], [3, 4]] and prm.digits(2) == [[0, 1]]
    h = 8
    s, keys, emax = _keys_and_secret(prm, 31, 7, (5, 1), h)
    for level in (7, 6, 4, 3, 1):
        ct = ki.ciphertexts(31, prm.q[:level], prm.N, 1)[0]
        for key in keys:
            out = ks.keyswitch(prm, ct, key, level)
            _check_decrypts(prm, ct, out, s, key.galois, level, emax, h)


def test_partitions_agree_at_the_top_level():
    """At level L both partitions have the same digits and keys: the same bits."""
    p0, p1 = ks.Params(6, 6, 3, 2), ks.Params(6, 6, 3, 2, partition=1)
    s, (key,), _ = _keys_and_secret(p0, 32, 6, (5,), 8)
    ct = ki.ciphertexts(32, p0.q, p0.N, 1)[0]
    assert np.array_equal(ks.keyswitch(p0, ct, key, 6), ks.keyswitch(p1, ct, key, 6))


def test_top_level_partition_needs_the_key_basis_index(monkeypatch):
    """Reading the special-prime limbs of a top-level key at the ciphertext's own
    index (as a level-l key would be read) breaks the key switch below L."""
    prm = ks.Params(6, 6, 3, 2, partition=1)
    s, (key,), emax = _keys_and_secret(prm, 33, 6, (5,), 8)
    level = 4
    ct = ki.ciphertexts(33, prm.q[:level], prm.N, 1)[0]
    _check_decrypts(prm, ct, ks.keyswitch(prm, ct, key, level), s, 5, level, emax, 8)
    monkeypatch.setattr(ks.Params, "key_limb", lambda self, level, j: j)
    out = ks.keyswitch(prm, ct, key, level)
    e = ks.decryption_error(prm, ct, out, s, 5, level)
    assert e is None or np.abs(e).max() > ks.error_bound(prm, level, emax, 8)


@pytest.mark.parametrize("L,dnum,K,h", [(6, 3, 2, 8), (5, 2, 3, 12), (4, 4, 1, 4)])
def test_error_bound_is_reached_by_a_worst_case_input(L, dnum, K, h):
    """The bound holds and is nearly attained, so a dropped or extra factor fails.

    Every coefficient of c1 is the integer whose residue on each q_i of digit D
    is [-(Q_d/q_i)]_{q_i}. Fast base conversion then sums alpha_d terms
    (q_i - 1) Q_d/q_i, so every ModUp coefficient is alpha_d Q_d - sum_i Q_d/q_i,
    the top of its range. With every key error equal to E_max, coefficient N-1
    of ext_d * e_d adds N equal positive terms (no negacyclic wrap reaches it),
    and after the division by P the error there is
    sum_d N alpha_d (Q_d/P) E_max up to the ModDown term, which lies in
    [-K h, K (1 + h)] by the floor form's range [0, K P) per coefficient.
    """
    prm = small_params(log2n=6, L=L, dnum=dnum, K=K)
    N, level, emax = prm.N, L, 19
    digits = prm.digits(level)
    c1 = np.empty((level, N), dtype=np.uint64)
    for D in digits:
        Qd = math.prod(prm.q[i] for i in D)
        for i in D:
            c1[i] = rns.ntt(np.full(N, (-(Qd // prm.q[i])) % prm.q[i], dtype=np.uint64), prm.q[i])
    ct = np.stack([np.zeros_like(c1), c1])
    s = ki.ternary_secret(L * 100 + K, N, h)
    errs = np.full((len(digits), N), emax, dtype=np.int64)
    key = ks.keygen(prm, s, errs, ki.key_seed(L, K), level, 1)
    out = ks.keyswitch(prm, ct, key, level)
    e = ks.decryption_error(prm, ct, out, s, 1, level)
    assert e is not None
    B = ks.error_bound(prm, level, emax, h)
    assert np.abs(e).max() <= B
    assert int(np.argmax(e)) == N - 1
    assert e[N - 1] >= B - 2 * K * (1 + h) - 1
    # the top term alone is a large share of the bound (the bound is not loose)
    assert B - K * (1 + h) > 50 * K * (1 + h)


def test_planted_mistakes_fail_the_decryption_check(monkeypatch):
    """Mistakes planted in the oracle (on the CPU) must break the decryption check."""
    prm = small_params(log2n=6, L=4, dnum=2, K=2)
    level = 4
    s, (key,), emax = _keys_and_secret(prm, 11, level, (5,), 8)
    ct = ki.ciphertexts(11, prm.q, prm.N, 1)[0]
    good = ks.keyswitch(prm, ct, key, level)
    _check_decrypts(prm, ct, good, s, 5, level, emax, 8)
    B = ks.error_bound(prm, level, emax, 8)

    def fails(out):
        e = ks.decryption_error(prm, ct, out, s, 5, level)
        return e is None or np.abs(e).max() > B

    # dropped c0 term
    bad = good.copy()
    bad[0] = ks.moddown(prm, ks.inner_product(prm, ks.modup(prm, ct[1], level), key, level)[0], level)
    assert fails(bad)
    # one limb of the output off by one
    bad = good.copy()
    bad[1, 2, 7] = (int(bad[1, 2, 7]) + 1) % prm.q[2]
    assert fails(bad)
    # a digit dropped from the inner product
    ext = ks.modup(prm, ct[1], level)
    ext[1] = 0
    assert fails(ks.keyswitch_from_ext(prm, ct, ext, key, level))
    # a transposed automorphism (inverse map instead of the forward one)
    real = ks.automorphism_index
    monkeypatch.setattr(ks, "automorphism_index", lambda N, k: np.argsort(real(N, k)))
    bad = ks.keyswitch(prm, ct, key, level)
    monkeypatch.setattr(ks, "automorphism_index", real)
    assert fails(bad)
    # the wrong special-prime scale in ModDown
    with monkeypatch.context() as m:
        m.setattr(ks.Params, "P", property(lambda self: math.prod(self.p) + 2))
        bad = ks.keyswitch(prm, ct, key, level)
    assert fails(bad)


@pytest.mark.slow
def test_full_size_relinearisation_decrypts():
    w = ki.WORKLOADS["n16"]
    prm = ks.Params(w.log2n, w.L, w.dnum, w.K)
    s, (key,), emax = _keys_and_secret(prm, w.index, w.L, (1,), w.h)
    ct = ki.ciphertexts(w.index, prm.q, prm.N, 1)[0]
    out = ks.keyswitch(prm, ct, key, w.L)
    _check_decrypts(prm, ct, out, s, 1, w.L, emax, w.h)
