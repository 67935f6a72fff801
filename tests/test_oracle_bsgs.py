"""Pins of the oracle's double-hoisted BSGS linear transform (CPU only).

* Special cases reduce to operations pinned elsewhere: the identity diagonal
  returns the ciphertext exactly; a single baby step, and a single giant step,
  with a unit diagonal return exactly the pinned key switch of that rotation.
* In general the output decrypts, within an analytic bound, to
  sum_j phi_{G_j}(sum_i pt[j][i] phi_{g_i}(m)) computed directly on the
  message with small integer plaintexts.
* Planted mistakes (the P factor dropped from the baby steps, the giant
  rotation of inner_j,0 dropped, the diagonals transposed) must fail.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

import ks_inputs as ki
from oracle import bsgs
from oracle import keyswitch as ks
from oracle import rns

U64 = np.uint64


def _params():
    return ks.Params(12, 7, 3, 3)


def _keys(prm, widx, s, level, galois_list, first=0):
    keys, emax = [], 0
    for k, g in enumerate(galois_list):
        errs = ki.gaussian_errors(widx, first + k, len(prm.digits(level)), prm.N)
        emax = max(emax, int(np.abs(errs).max()))
        keys.append(ks.keygen(prm, s, errs, ki.key_seed(widx, first + k), level, g))
    return keys, emax


def _const_diag(prm, level, n2, n1, values):
    """diag[j][i] = the constant values[j][i] on every limb and position."""
    d = np.zeros((n2, n1, level + prm.K, prm.N), dtype=U64)
    for j in range(n2):
        for i in range(n1):
            for t, r in enumerate(prm.basis(level)):
                d[j, i, t] = U64(values[j][i] % r)
    return d


def test_identity_diagonal_returns_the_ciphertext():
    prm = _params()
    level = 5
    ct = ki.ciphertexts(120, prm.q[:level], prm.N, 1)[0]
    out = bsgs.linear_transform(prm, ct, _const_diag(prm, level, 1, 1, [[1]]), [], [], level)
    assert np.array_equal(out, ct.astype(U64))


@pytest.mark.parametrize("level", [7, 4])
def test_single_baby_step_is_the_key_switch(level):
    prm = _params()
    s = ki.ternary_secret(121, prm.N, 32)
    (key,), _ = _keys(prm, 121, s, level, [5])
    ct = ki.ciphertexts(121, prm.q[:level], prm.N, 1)[0]
    out = bsgs.linear_transform(prm, ct, _const_diag(prm, level, 1, 2, [[0, 1]]), [key], [], level)
    assert np.array_equal(out, ks.keyswitch(prm, ct, key, level))


@pytest.mark.parametrize("level", [7, 3])
def test_single_giant_step_is_the_key_switch(level):
    prm = _params()
    s = ki.ternary_secret(122, prm.N, 32)
    (key,), _ = _keys(prm, 122, s, level, [25])
    ct = ki.ciphertexts(122, prm.q[:level], prm.N, 1)[0]
    out = bsgs.linear_transform(prm, ct, _const_diag(prm, level, 2, 1, [[0], [1]]), [], [key], level)
    assert np.array_equal(out, ks.keyswitch(prm, ct, key, level))


def _bound(prm, level, n1, n2, emax, h, pt_bound):
    """Coefficient bound on the transform's error (see the module docstring of oracle.bsgs).

    Each baby step carries the key-switching error B (after the division by P),
    multiplied by a plaintext: at most N * pt_bound * B per step. Each giant
    step adds the floor error of ModDown(inner_j,1) times s (at most (K+1) h),
    its own key switch (B), and the final ModDown adds at most K (1 + h).
    """
    B = ks.error_bound(prm, level, emax, h)
    per_giant = n1 * prm.N * pt_bound * B + (prm.K + 1) * h + B
    return n2 * per_giant + prm.K * (1 + h)


def _error(prm, out, expected, s, level):
    sh = ks.secret_eval(prm, s, level)
    lifts = []
    for i in range(level):
        q = U64(prm.q[i])
        dec = (out[0, i] + out[1, i] * sh[i] % q) % q
        lifts.append(rns.centered(rns.intt((dec + (q - expected[i])) % q, prm.q[i]), prm.q[i]))
    if any(not np.array_equal(x, lifts[0]) for x in lifts[1:]):
        return None
    return lifts[0]


def _random_case(widx, level, n1, n2, pt_bound=3, h=32):
    prm = _params()
    s = ki.ternary_secret(widx, prm.N, h)
    baby_g = [ki.galois_rot(i, prm.N) for i in range(1, n1)]
    giant_g = [ki.galois_rot(j * n1, prm.N) for j in range(1, n2)]
    baby, e1 = _keys(prm, widx, s, level, baby_g)
    giant, e2 = _keys(prm, widx, s, level, giant_g, first=len(baby_g))
    ct = ki.ciphertexts(widx, prm.q[:level], prm.N, 1)[0]
    coeffs = ki.small_plaintexts(widx, n1 * n2, prm.N, pt_bound)
    diag = np.stack([np.stack([bsgs.plaintext_eval(prm, coeffs[j * n1 + i], level) for i in range(n1)])
                     for j in range(n2)])
    expected = bsgs.expected_message(prm, ct, s, diag, baby_g, giant_g, level)
    bound = _bound(prm, level, n1, n2, max(e1, e2), h, pt_bound)
    return prm, ct, diag, baby, giant, s, expected, bound


@pytest.mark.parametrize("level,n1,n2", [(7, 3, 3), (5, 2, 3), (4, 4, 1)])
def test_decrypts_to_the_transformed_message(level, n1, n2):
    prm, ct, diag, baby, giant, s, expected, bound = _random_case(130 + level, level, n1, n2)
    out = bsgs.linear_transform(prm, ct, diag, baby, giant, level)
    e = _error(prm, out, expected, s, level)
    assert e is not None, "error residues differ between limbs"
    assert np.abs(e).max() <= bound
    # the bound is far below Q/2, so a wrong transform cannot pass by wrapping
    assert bound < Fraction(math.prod(prm.q[:level]), 2 ** 20)


def test_planted_mistakes_fail(monkeypatch):
    level, n1, n2 = 6, 2, 2
    prm, ct, diag, baby, giant, s, expected, bound = _random_case(140, level, n1, n2)

    def fails(out):
        e = _error(prm, out, expected, s, level)
        return e is None or np.abs(e).max() > bound

    good = bsgs.linear_transform(prm, ct, diag, baby, giant, level)
    assert not fails(good)
    # baby steps without the factor P on the c0 and identity terms
    with monkeypatch.context() as m:
        m.setattr(bsgs, "scale_by_p", lambda prm_, c, lv: np.concatenate(
            [np.asarray(c, dtype=U64), np.zeros((prm_.K, prm_.N), dtype=U64)]))
        assert fails(bsgs.linear_transform(prm, ct, diag, baby, giant, level))
    # giant steps that forget to rotate inner_j,0
    with monkeypatch.context() as m:
        m.setattr(bsgs, "giant_rotation", lambda x, g: np.array(x, copy=True))
        assert fails(bsgs.linear_transform(prm, ct, diag, baby, giant, level))
    # the diagonals indexed [baby][giant] instead of [giant][baby]
    assert fails(bsgs.linear_transform(prm, ct, np.ascontiguousarray(diag.transpose(1, 0, 2, 3)), baby, giant,
                                       level))
