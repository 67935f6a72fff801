"""Double-hoisted baby-step/giant-step linear transform (oracle; test infrastructure only).

The pages place key switching under the bootstrap's linear transforms: the
hoisted-rotation workload is described as shaped like a baby-step/giant-step
stage of a bootstrap, and the Perseus README ('Runtime') times bootstraps
with the runtime's primitives. They do not write the transform down, so this
module follows the textbook double-hoisted evaluation, step by step, for one
ciphertext ct = (c0, c1) at level l, n1 baby steps with Galois elements
g_0 = 1, g_1..g_{n1-1} and n2 giant steps with G_0 = 1, G_1..G_{n2-1}, and
plaintext diagonals pt[j][i] given over the extended basis q_0..q_{l-1},
p_0..p_{K-1} in evaluation form:

1. ModUp of c1, once (first hoisting).
2. Baby step i in the extended basis, with no ModDown:
   R_i = (P phi_{g_i}(c0) + IP_0, IP_1), IP = the inner product of
   phi_{g_i}(ext) with the key of g_i; R_0 = (P c0, P c1). P times a q-limb is
   [P]_{q} times it; P vanishes on the p-limbs.
3. Per giant step j: inner_j = sum_i pt[j][i] R_i, limb by limb (second
   hoisting: the baby steps are summed before any ModDown).
4. acc = inner_0 + sum_{j>=1} (phi_{G_j}(inner_j,0) + KS_j), where KS_j is the
   inner product of phi_{G_j}(ModUp(ModDown(inner_j,1))) with the key of G_j;
   the only ModDown per giant step is that of inner_j's second component.
5. out = ModDown of both components of acc.

Up to key-switching noise, out decrypts to
sum_j phi_{G_j}(sum_i pt[j][i] phi_{g_i}(m)) for m the message of ct. The
reading of steps 2-4 (where P enters, that phi_{G_j} acts on inner_j,0 in the
extended basis) is listed in the design notes.
"""

from __future__ import annotations

import numpy as np

from . import keyswitch as ks

U64 = np.uint64


def scale_by_p(prm: ks.Params, c: np.ndarray, level: int) -> np.ndarray:
    """[l][N] over Q -> [l+K][N] over Q u P: P c on the q-limbs, 0 on the p-limbs."""
    out = np.zeros((level + prm.K, prm.N), dtype=U64)
    for i in range(level):
        q = prm.q[i]
        out[i] = np.asarray(c[i], dtype=U64) * U64(prm.P % q) % U64(q)
    return out


def baby_steps(prm: ks.Params, ct: np.ndarray, baby_keys: list, level: int) -> list:
    """[R_0, ..., R_{n1-1}], each [2][l+K][N] in the extended basis (one shared ModUp)."""
    ct = np.asarray(ct, dtype=U64)
    basis = prm.basis(level)
    steps = [np.stack([scale_by_p(prm, ct[0], level), scale_by_p(prm, ct[1], level)])]
    if not baby_keys:
        return steps
    ext = ks.modup(prm, ct[1], level)
    for key in baby_keys:
        acc = ks.inner_product(prm, ext, key, level)
        pc0 = scale_by_p(prm, ks.automorphism(ct[0], key.galois), level)
        for j, r in enumerate(basis):
            acc[0, j] = (acc[0, j] + pc0[j]) % U64(r)
        steps.append(acc)
    return steps


def giant_sum(prm: ks.Params, steps: list, diag: np.ndarray, j: int, level: int) -> np.ndarray:
    """inner_j [2][l+K][N] = sum_i diag[j][i] R_i, limb by limb."""
    basis = prm.basis(level)
    inner = np.zeros((2, len(basis), prm.N), dtype=U64)
    for i, R in enumerate(steps):
        for jj, r in enumerate(basis):
            pt = np.asarray(diag[j, i, jj], dtype=U64)
            for u in range(2):
                inner[u, jj] = (inner[u, jj] + pt * R[u, jj] % U64(r)) % U64(r)
    return inner


def giant_rotation(x: np.ndarray, galois: int) -> np.ndarray:
    """phi_{G_j} of inner_j,0, applied in the extended basis (limb by limb, evaluation form)."""
    return ks.automorphism(x, galois)


def linear_transform(prm: ks.Params, ct: np.ndarray, diag: np.ndarray, baby_keys: list, giant_keys: list,
                     level: int) -> np.ndarray:
    """out [2][l][N]; diag [n2][n1][l+K][N] with n1 = 1 + len(baby_keys), n2 = 1 + len(giant_keys)."""
    diag = np.asarray(diag, dtype=U64)
    n2, n1 = diag.shape[0], diag.shape[1]
    if n1 != 1 + len(baby_keys) or n2 != 1 + len(giant_keys):
        raise ValueError("diag must be [1 + giant keys][1 + baby keys][l+K][N]")
    basis = prm.basis(level)
    steps = baby_steps(prm, ct, baby_keys, level)
    acc = giant_sum(prm, steps, diag, 0, level)
    for j, key in enumerate(giant_keys, start=1):
        inner = giant_sum(prm, steps, diag, j, level)
        d1 = ks.moddown(prm, inner[1], level)
        ks_j = ks.inner_product(prm, ks.modup(prm, d1, level), key, level)
        rot0 = giant_rotation(inner[0], key.galois)
        for jj, r in enumerate(basis):
            R = U64(r)
            acc[0, jj] = (acc[0, jj] + rot0[jj] + ks_j[0, jj]) % R
            acc[1, jj] = (acc[1, jj] + ks_j[1, jj]) % R
    return np.stack([ks.moddown(prm, acc[0], level), ks.moddown(prm, acc[1], level)])


def plaintext_eval(prm: ks.Params, coeffs: np.ndarray, level: int) -> np.ndarray:
    """[l+K][N] evaluation form of an integer polynomial over the extended basis."""
    return ks.secret_eval(prm, coeffs, level)


def expected_message(prm: ks.Params, ct: np.ndarray, s: np.ndarray, diag: np.ndarray, baby_galois: list,
                     giant_galois: list, level: int) -> np.ndarray:
    """[l][N] evaluation form over Q of sum_j phi_{G_j}(sum_i pt[j][i] phi_{g_i}(c0 + c1 s))."""
    ct = np.asarray(ct, dtype=U64)
    diag = np.asarray(diag, dtype=U64)
    sh = ks.secret_eval(prm, s, level)
    m = np.stack([(ct[0, i] + ct[1, i] * sh[i] % U64(prm.q[i])) % U64(prm.q[i]) for i in range(level)])
    gs = [1] + list(baby_galois)
    Gs = [1] + list(giant_galois)
    total = np.zeros((level, prm.N), dtype=U64)
    for j, G in enumerate(Gs):
        inner = np.zeros((level, prm.N), dtype=U64)
        for i, g in enumerate(gs):
            mr = ks.automorphism(m, g)
            for t in range(level):
                q = U64(prm.q[t])
                inner[t] = (inner[t] + diag[j, i, t] * mr[t] % q) % q
        rot = ks.automorphism(inner, G)
        for t in range(level):
            total[t] = (total[t] + rot[t]) % U64(prm.q[t])
    return total
