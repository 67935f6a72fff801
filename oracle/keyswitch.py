"""RNS-CKKS hybrid key switching, step by step (oracle; test infrastructure only).

The pages name the operation and its regenerated key half (Perseus README,
'What's inside' and 'Layout'; arXiv summary page, methodology item (i)) but
do not write the algorithm down. This module follows the textbook hybrid key
switch with fast base conversion, in this order, for one ciphertext (c0, c1)
at level l (l active ciphertext primes) and a key with Galois element k
(k = 1: no automorphism, the relinearisation case):

1. c1 to coefficients, limb by limb (inverse NTT).
2. ModUp per digit D_d: y_i = [c1_i * (Q_d/q_i)^-1]_{q_i} for i in D_d and,
   for every other modulus t of the basis q_0..q_{l-1}, p_0..p_{K-1},
   z_t = (sum_i y_i * [Q_d/q_i]_t) mod t, taken back to evaluation form; the
   digit's own limbs are c1's limbs as given.
3. Automorphism of every extended limb in evaluation form:
   ext'[i] = ext[(i*k + (k-1)/2) mod N].
4. Inner product with the key over all l+K limbs:
   acc0 = sum_d ext'_d * b_d, acc1 = sum_d ext'_d * a_d (mod r_j), where a_d
   comes from the ChaCha expander or a stored array.
5. ModDown of each acc_u: x_t = iNTT(acc_u on p_t), y_t = [x_t (P/p_t)^-1]_{p_t},
   z_i = (sum_t y_t [P/p_t]_{q_i}) mod q_i,
   out_u[i] = (acc_u[i] - NTT(z_i)) * [P^-1]_{q_i} mod q_i  (floor form, no
   rounding term).
6. out0 += the automorphism of c0.

Readings where the pages are silent:
by default (partition 0) digits at level l have alpha(l) = ceil(l/dnum)
primes each, D_d = [d*alpha, min((d+1)*alpha, l)), and the key is generated at
level l; with partition 1 alpha = ceil(L/dnum) at every level, the digits are
those of the top level cut at l, and one key generated at level L serves every
level (its limbs q_l..q_{L-1} are not used); a key's limb is indexed in the key
basis (q limbs first, then p limbs), so at level l limb j of the extended basis
is key limb j for j < l and key_level + (j - l) for the special primes; the key
equation is b_d = -a_d s + e_d + g_d s' with g_d = [P]_{q_j} on the q-limbs of
D_d and 0 elsewhere; decryption is c0 + c1 s.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from fractions import Fraction

import numpy as np

from . import chacha
from .rns import centered, find_psi, intt, ntt, ntt_primes, to_residues

U64 = np.uint64


@dataclass
class Params:
    log2n: int
    L: int
    dnum: int
    K: int
    primes: tuple = None  # L q-primes then K p-primes; default: the descending rule
    chacha_rounds: int = 12
    partition: int = 0    # 0: alpha(l) = ceil(l/dnum), key at level l; 1: alpha = ceil(L/dnum), key at level L

    def __post_init__(self):
        if self.primes is None:
            self.primes = tuple(ntt_primes(self.N, self.L + self.K))
        self.primes = tuple(int(p) for p in self.primes)
        assert len(self.primes) == self.L + self.K
        for p in self.primes:
            find_psi(p, self.N)  # also asserts p = 1 mod 2N

    @property
    def N(self) -> int:
        return 1 << self.log2n

    @property
    def q(self) -> tuple:
        return self.primes[: self.L]

    @property
    def p(self) -> tuple:
        return self.primes[self.L:]

    @property
    def P(self) -> int:
        return math.prod(self.p)

    def alpha(self, level: int) -> int:
        return -(-(self.L if self.partition else level) // self.dnum)

    def key_level(self, level: int) -> int:
        """Level of the key that serves ciphertexts at ``level``."""
        return self.L if self.partition else level

    def key_limb(self, level: int, j: int) -> int:
        """Key-basis index of limb j of the extended basis at ``level``."""
        return j if j < level else self.key_level(level) + (j - level)

    def digits(self, level: int) -> list:
        """Index lists D_0..D_{beta-1} of the q-limbs at this level."""
        a = self.alpha(level)
        return [list(range(s, min(s + a, level))) for s in range(0, level, a)]

    def basis(self, level: int) -> list:
        """Moduli of the extended basis: q_0..q_{level-1}, p_0..p_{K-1}."""
        return list(self.q[:level]) + list(self.p)


# ---------------------------------------------------------------------------
# step 1-2: ModUp
# ---------------------------------------------------------------------------

def modup(prm: Params, c1: np.ndarray, level: int) -> np.ndarray:
    """c1 [l][N] (evaluation form) -> ext [beta][l+K][N] (evaluation form)."""
    c1 = np.asarray(c1, dtype=U64)
    N = prm.N
    basis = prm.basis(level)
    coef = [intt(c1[i], prm.q[i]) for i in range(level)]
    digits = prm.digits(level)
    ext = np.empty((len(digits), level + prm.K, N), dtype=U64)
    for d, D in enumerate(digits):
        Qd = math.prod(prm.q[i] for i in D)
        y = {}
        for i in D:
            qi = prm.q[i]
            qhat = Qd // qi
            y[i] = coef[i] * U64(pow(qhat % qi, -1, qi)) % U64(qi)
        for j, t in enumerate(basis):
            if j in D:
                ext[d, j] = c1[j]
                continue
            z = np.zeros(N, dtype=U64)
            for i in D:
                z = (z + y[i] * U64((Qd // prm.q[i]) % t) % U64(t)) % U64(t)
            ext[d, j] = ntt(z, t)
    return ext


# ---------------------------------------------------------------------------
# step 3: automorphism
# ---------------------------------------------------------------------------

def automorphism_index(N: int, k: int) -> np.ndarray:
    """Evaluation-domain source index of X -> X^k: i -> (i*k + (k-1)/2) mod N."""
    if k % 2 == 0:
        raise ValueError("Galois element must be odd")
    i = np.arange(N, dtype=np.int64)
    return (i * k + (k - 1) // 2) % N


def automorphism(x: np.ndarray, k: int) -> np.ndarray:
    """Apply X -> X^k to evaluation-form limbs (last axis)."""
    if k == 1:
        return np.array(x, copy=True)
    return np.asarray(x)[..., automorphism_index(np.asarray(x).shape[-1], k)]


# ---------------------------------------------------------------------------
# step 4: the key and the inner product
# ---------------------------------------------------------------------------

@dataclass
class Key:
    """A key-switching key at level ``level`` for Galois element ``galois``.

    b: [beta][level+K][N] evaluation form. The a half is either regenerated
    from ``seed`` (32 bytes) or given in ``a`` with the same shape as b.
    """
    b: np.ndarray
    seed: bytes
    level: int
    galois: int = 1
    a: np.ndarray = None


def key_a(prm: Params, key: Key) -> np.ndarray:
    """The a half of a key: stored, or expanded from its seed (limb j = key-basis index)."""
    if key.a is not None:
        return np.asarray(key.a, dtype=U64)
    basis = prm.basis(key.level)
    beta = len(prm.digits(key.level))
    out = np.empty((beta, len(basis), prm.N), dtype=U64)
    for d in range(beta):
        for j, r in enumerate(basis):
            out[d, j] = chacha.expand_uniform(key.seed, d, j, prm.N, r, prm.chacha_rounds)
    return out


def inner_product(prm: Params, ext: np.ndarray, key: Key, level: int) -> np.ndarray:
    """acc [2][l+K][N]: sum over digits of automorphism(ext_d) times (b_d, a_d)."""
    if key.level != prm.key_level(level):
        raise ValueError(f"this partition needs a key at level {prm.key_level(level)}")
    basis = prm.basis(level)
    a = key_a(prm, key)
    b = np.asarray(key.b, dtype=U64)
    acc = np.zeros((2, len(basis), prm.N), dtype=U64)
    for d in range(ext.shape[0]):
        e = automorphism(ext[d], key.galois)
        for j, r in enumerate(basis):
            kj = prm.key_limb(level, j)
            acc[0, j] = (acc[0, j] + e[j] * b[d, kj] % U64(r)) % U64(r)
            acc[1, j] = (acc[1, j] + e[j] * a[d, kj] % U64(r)) % U64(r)
    return acc


# ---------------------------------------------------------------------------
# step 5: ModDown
# ---------------------------------------------------------------------------

def moddown(prm: Params, acc: np.ndarray, level: int) -> np.ndarray:
    """acc [l+K][N] (evaluation form, basis Q_l u P) -> [l][N] = (acc - Conv_P->Q([acc]_P)) / P."""
    acc = np.asarray(acc, dtype=U64)
    P = prm.P
    y = []
    for t, pt in enumerate(prm.p):
        x = intt(acc[level + t], pt)
        y.append(x * U64(pow((P // pt) % pt, -1, pt)) % U64(pt))
    out = np.empty((level, prm.N), dtype=U64)
    for i in range(level):
        qi = prm.q[i]
        z = np.zeros(prm.N, dtype=U64)
        for t, pt in enumerate(prm.p):
            z = (z + y[t] * U64((P // pt) % qi) % U64(qi)) % U64(qi)
        zh = ntt(z, qi)
        diff = (acc[i] + (U64(qi) - zh)) % U64(qi)
        out[i] = diff * U64(pow(P % qi, -1, qi)) % U64(qi)
    return out


# ---------------------------------------------------------------------------
# the whole key switch
# ---------------------------------------------------------------------------

def keyswitch_from_ext(prm: Params, ct: np.ndarray, ext: np.ndarray, key: Key, level: int) -> np.ndarray:
    """Steps 3-6 for one key, given the ModUp output of ct's c1."""
    acc = inner_product(prm, ext, key, level)
    out = np.empty((2, level, prm.N), dtype=U64)
    out[0] = moddown(prm, acc[0], level)
    out[1] = moddown(prm, acc[1], level)
    c0 = automorphism(np.asarray(ct[0], dtype=U64), key.galois)
    for i in range(level):
        out[0, i] = (out[0, i] + c0[i]) % U64(prm.q[i])
    return out


def keyswitch(prm: Params, ct: np.ndarray, key: Key, level: int) -> np.ndarray:
    """One key switch of ct [2][l][N] -> [2][l][N] (uint64 residues)."""
    ext = modup(prm, ct[1], level)
    return keyswitch_from_ext(prm, ct, ext, key, level)


def keyswitch_hoisted(prm: Params, ct: np.ndarray, keys: list, level: int) -> np.ndarray:
    """ModUp once, then steps 3-6 per key: [R][2][l][N]."""
    ext = modup(prm, ct[1], level)
    return np.stack([keyswitch_from_ext(prm, ct, ext, k, level) for k in keys])


# ---------------------------------------------------------------------------
# key generation and the decryption check (test support)
# ---------------------------------------------------------------------------

def secret_eval(prm: Params, s: np.ndarray, level: int) -> np.ndarray:
    """[l+K][N] evaluation form of an integer polynomial over the basis at ``level``."""
    return np.stack([ntt(to_residues(s, r), r) for r in prm.basis(level)])


def target_secret_eval(prm: Params, s: np.ndarray, galois: int, level: int) -> np.ndarray:
    """Evaluation form of s': s^2 for the relinearisation key (galois 1), phi_k(s) otherwise."""
    sh = secret_eval(prm, s, level)
    if galois == 1:
        basis = prm.basis(level)
        return np.stack([sh[j] * sh[j] % U64(r) for j, r in enumerate(basis)])
    return automorphism(sh, galois)


def keygen(prm: Params, s: np.ndarray, errors: np.ndarray, seed: bytes, level: int, galois: int) -> Key:
    """b_d[j] = -a_d[j] s[j] + e_d[j] + g_{d,j} s'[j] (mod r_j), evaluation form.

    g_{d,j} = [P]_{q_j} when j is a q-limb of digit d, else 0. ``errors`` holds one
    integer polynomial per digit.
    """
    basis = prm.basis(level)
    digits = prm.digits(level)
    key = Key(b=None, seed=seed, level=level, galois=galois)
    a = key_a(prm, key)
    sh = secret_eval(prm, s, level)
    s2 = target_secret_eval(prm, s, galois, level)
    b = np.empty_like(a)
    for d, D in enumerate(digits):
        for j, r in enumerate(basis):
            R = U64(r)
            eh = ntt(to_residues(errors[d], r), r)
            g = U64(prm.P % r) if j in D else U64(0)
            b[d, j] = ((R - a[d, j] * sh[j] % R) + eh + g * s2[j] % R) % R
    key.b = b
    return key


def error_bound(prm: Params, level: int, e_max: int, h: int) -> Fraction:
    """B = sum_d N alpha_d (Q_d/P) E_max + K (1 + h) on the key-switching error."""
    P = prm.P
    B = Fraction(0)
    for D in prm.digits(level):
        Qd = math.prod(prm.q[i] for i in D)
        B += Fraction(prm.N * len(D) * Qd * e_max, P)
    return B + prm.K * (1 + h)


def decryption_error(prm: Params, ct: np.ndarray, out: np.ndarray, s: np.ndarray, galois: int, level: int):
    """Key-switching error polynomial, or None if its residues disagree across limbs.

    e = out0 + out1 s - (phi(c0) + phi(c1) s') (mod Q_l), lifted limb by limb to
    (-q/2, q/2]; a genuine small error has the same lift on every limb.
    """
    sh = secret_eval(prm, s, level)
    s2 = target_secret_eval(prm, s, galois, level)
    c = automorphism(np.asarray(ct, dtype=U64), galois)
    lifts = []
    for i in range(level):
        qi = U64(prm.q[i])
        lhs = (np.asarray(out[0, i], dtype=U64) + np.asarray(out[1, i], dtype=U64) * sh[i] % qi) % qi
        rhs = (c[0, i] + c[1, i] * s2[i] % qi) % qi
        diff = (lhs + (qi - rhs)) % qi
        lifts.append(centered(intt(diff, prm.q[i]), prm.q[i]))
    for x in lifts[1:]:
        if not np.array_equal(x, lifts[0]):
            return None
    return lifts[0]
