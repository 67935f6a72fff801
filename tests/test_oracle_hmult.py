"""Pins of the oracle's homomorphic multiplication (CPU only).

* The tensor product is checked against negacyclic schoolbook products of the
  coefficient polynomials (a different route from the pointwise evaluation-form
  products), and against the decryption identity
  d0 + d1 s + d2 s^2 = (a0 + a1 s)(b0 + b1 s).
* Rescaling is checked coefficient by coefficient against big integers: the
  CRT lift C over Q_l must give round(C / q_{l-1}) mod every remaining prime.
* Relinearisation is the key switch of (d0, d2), checked by decryption within
  the analytic bound.
* Planted mistakes (a dropped cross term, a truncating rescale) must fail.
"""

import math

import numpy as np
import pytest
from sympy.ntheory.modular import crt

import ks_inputs as ki
from oracle import hmult as hm
from oracle import keyswitch as ks
from oracle import rns


def _params():
    return ks.Params(6, 4, 2, 2)


def _negacyclic(a, b, q):
    """Schoolbook product mod X^N + 1 (Python integers)."""
    N = len(a)
    out = [0] * N
    for i in range(N):
        ai = int(a[i])
        for j in range(N):
            v = ai * int(b[j])
            if i + j < N:
                out[i + j] += v
            else:
                out[i + j - N] -= v
    return np.array([x % q for x in out], dtype=np.uint64)


def test_tensor_matches_schoolbook_products():
    prm = _params()
    level = 3
    a, b = ki.ciphertexts(70, prm.q[:level], prm.N, 2)
    d = hm.tensor(prm, a, b, level)
    for i in range(level):
        q = prm.q[i]
        ac = [rns.intt(a[u, i], q) for u in range(2)]
        bc = [rns.intt(b[u, i], q) for u in range(2)]
        d0 = _negacyclic(ac[0], bc[0], q)
        d1 = (_negacyclic(ac[0], bc[1], q) + _negacyclic(ac[1], bc[0], q)) % np.uint64(q)
        d2 = _negacyclic(ac[1], bc[1], q)
        for k, ref in enumerate((d0, d1, d2)):
            assert np.array_equal(rns.intt(d[k, i], q), ref), (k, i)


def _product_identity_holds(prm, d, a, b, sh, level):
    for i in range(level):
        q = np.uint64(prm.q[i])
        lhs = (d[0, i] + d[1, i] * sh[i] % q + d[2, i] * (sh[i] * sh[i] % q) % q) % q
        rhs = (a[0, i] + a[1, i] * sh[i] % q) % q * ((b[0, i] + b[1, i] * sh[i] % q) % q) % q
        if not np.array_equal(lhs, rhs):
            return False
    return True


def test_tensor_decrypts_to_the_product():
    prm = _params()
    level = 4
    sh = ks.secret_eval(prm, ki.ternary_secret(71, prm.N, 8), level)
    a, b = ki.ciphertexts(71, prm.q, prm.N, 2)
    assert _product_identity_holds(prm, hm.tensor(prm, a, b, level), a, b, sh, level)


def _rescale_rounds(prm, ct, out, level):
    ql = prm.q[level - 1]
    Q = math.prod(prm.q[:level])
    for u in range(ct.shape[0]):
        coef = [rns.intt(ct[u, i], prm.q[i]) for i in range(level)]
        ocoef = [rns.intt(out[u, i], prm.q[i]) for i in range(level - 1)]
        for n in range(prm.N):
            C = int(crt(list(prm.q[:level]), [int(coef[i][n]) for i in range(level)])[0]) % Q
            D = (2 * C + ql) // (2 * ql)  # nearest integer to C / ql (no ties: ql is odd)
            for i in range(level - 1):
                if int(ocoef[i][n]) != D % prm.q[i]:
                    return False
    return True


@pytest.mark.parametrize("level", [4, 3, 2])
def test_rescale_rounds_the_crt_lift(level):
    prm = _params()
    ct = ki.ciphertexts(72 + level, prm.q[:level], prm.N, 1)[0]
    assert _rescale_rounds(prm, ct, hm.rescale(prm, ct, level), level)


def test_hmult_relinearises_within_the_bound():
    prm = _params()
    level, h = 4, 8
    s = ki.ternary_secret(75, prm.N, h)
    errs = ki.gaussian_errors(75, 0, len(prm.digits(level)), prm.N)
    key = ks.keygen(prm, s, errs, ki.key_seed(75, 0), level, 1)
    a, b = ki.ciphertexts(75, prm.q, prm.N, 2)
    d = hm.tensor(prm, a, b, level)
    relin = hm.relinearise(prm, d, key, level)
    # (d0, d2) switched by the key of s^2 decrypts like d0 + d2 s^2
    ks_only = relin.copy()
    for i in range(level):
        q = np.uint64(prm.q[i])
        ks_only[1, i] = (relin[1, i] + (q - d[1, i])) % q
    e = ks.decryption_error(prm, np.stack([d[0], d[2]]), ks_only, s, 1, level)
    assert e is not None and np.abs(e).max() <= ks.error_bound(prm, level, int(np.abs(errs).max()), h)
    out = hm.hmult(prm, a, b, key, level)
    assert np.array_equal(out, hm.rescale(prm, relin, level))


def test_planted_mistakes_fail(monkeypatch):
    prm = _params()
    level = 3
    sh = ks.secret_eval(prm, ki.ternary_secret(76, prm.N, 8), level)
    a, b = ki.ciphertexts(76, prm.q[:level], prm.N, 2)
    # the tensor without the cross term a1 b0
    d = hm.tensor(prm, a, b, level)
    for i in range(level):
        q = np.uint64(prm.q[i])
        d[1, i] = a[0, i].astype(np.uint64) * b[1, i] % q
    assert not _product_identity_holds(prm, d, a, b, sh, level)
    # a rescale that truncates (no centring of the dropped limb)
    ct = ki.ciphertexts(77, prm.q[:level], prm.N, 1)[0]
    monkeypatch.setattr(hm, "centered", lambda x, q: np.asarray(x, dtype=np.int64))
    assert not _rescale_rounds(prm, ct, hm.rescale(prm, ct, level), level)
