"""Bit-exact parity of the GPU double-hoisted BSGS linear transform
(pc_linear_transform through the C ABI) with the oracle.

Small rings use real keys and small integer plaintext diagonals (the GPU output
then also decrypts to the transformed message); the N=2^16 workload uses uniform
key b halves with ChaCha seeds and uniform diagonals (bit-exactness does not
depend on either being meaningful).
"""

import numpy as np
import pytest

import ks_inputs as ki
from oracle import bsgs
from oracle import keyswitch as ks

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ksa = pytest.importorskip("key_switching_amd")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "these tests need the GPU"
    torch.cuda.set_device(0)
    yield 0
    torch.cuda.synchronize()


def dev(a):
    return ksa.to_device(a, 0)


def host(t):
    torch.cuda.synchronize()
    return ksa.to_host(t)


def assert_equal(gpu_words, oracle_words, what):
    g = np.asarray(gpu_words, dtype=np.uint64)
    o = np.asarray(oracle_words, dtype=np.uint64)
    assert g.shape == o.shape, (what, g.shape, o.shape)
    bad = np.flatnonzero(g.reshape(-1) != o.reshape(-1))
    assert bad.size == 0, f"{what}: {bad.size} of {g.size} words differ, first at flat index {bad[0]}"


def params_pair(log2n, L, dnum, K, **kw):
    prm = ksa.Params(log2n, L, dnum, K, device=0, **kw)
    oprm = ks.Params(log2n, L, dnum, K, partition=kw.get("partition", 0))
    assert tuple(prm.primes) == oprm.primes
    return prm, oprm


def _real_case(oprm, widx, level, n1, n2, h=32, pt_bound=3):
    kl = oprm.key_level(level)
    s = ki.ternary_secret(widx, oprm.N, h)
    baby_g = [ki.galois_rot(i, oprm.N) for i in range(1, n1)]
    giant_g = [ki.galois_rot(j * n1, oprm.N) for j in range(1, n2)]
    keys = []
    for k, g in enumerate(baby_g + giant_g):
        errs = ki.gaussian_errors(widx, k, len(oprm.digits(kl)), oprm.N)
        keys.append(ks.keygen(oprm, s, errs, ki.key_seed(widx, k), kl, g))
    baby, giant = keys[: n1 - 1], keys[n1 - 1:]
    ct = ki.ciphertexts(widx, oprm.q[:level], oprm.N, 1)[0]
    coeffs = ki.small_plaintexts(widx, n1 * n2, oprm.N, pt_bound)
    diag = np.stack([np.stack([bsgs.plaintext_eval(oprm, coeffs[j * n1 + i], level) for i in range(n1)])
                     for j in range(n2)])
    return ct, diag, baby, giant


def _run(prm, ct, diag, baby, giant, level):
    return host(ksa.linear_transform(
        prm, dev(ct), dev(diag), level,
        baby_b=[dev(k.b) for k in baby], baby_seeds=[k.seed for k in baby], baby_galois=[k.galois for k in baby],
        giant_b=[dev(k.b) for k in giant], giant_seeds=[k.seed for k in giant],
        giant_galois=[k.galois for k in giant]))


@pytest.mark.parametrize("level,n1,n2,partition", [
    (7, 3, 3, 0), (5, 2, 3, 0), (4, 4, 2, 0), (2, 1, 4, 0), (7, 3, 2, 1), (3, 2, 2, 1),
    (6, 8, 2, 0), (7, 1, 8, 0), (1, 2, 2, 0), (1, 3, 3, 1)])
def test_small_ring_matches_oracle(level, n1, n2, partition):
    """N=2^12, L=7, dnum=3, K=3 with real rotation keys and small diagonals."""
    prm, oprm = params_pair(12, 7, 3, 3, partition=partition, max_batch=4, max_hoist=8)
    ct, diag, baby, giant = _real_case(oprm, 150 + level + 10 * partition, level, n1, n2)
    out = _run(prm, ct, diag, baby, giant, level)
    assert_equal(out, bsgs.linear_transform(oprm, ct, diag, baby, giant, level), f"level {level} {n1}x{n2}")
    prm.close()


def _const_diag(oprm, level, values):
    n2, n1 = len(values), len(values[0])
    d = np.zeros((n2, n1, level + oprm.K, oprm.N), dtype=np.uint64)
    for j in range(n2):
        for i in range(n1):
            for t, r in enumerate(oprm.basis(level)):
                d[j, i, t] = values[j][i] % r
    return d


def test_special_cases_reduce_to_the_key_switch():
    """Identity diagonal: the ciphertext; a unit diagonal on one baby or one giant
    step: the GPU's own key switch by that rotation."""
    prm, oprm = params_pair(12, 7, 3, 3, max_batch=4, max_hoist=8)
    level = 6
    ct, _, baby, giant = _real_case(oprm, 170, level, 2, 2)
    same = _run(prm, ct, _const_diag(oprm, level, [[1]]), [], [], level)
    assert_equal(same, ct, "identity")
    one_baby = _run(prm, ct, _const_diag(oprm, level, [[0, 1]]), baby, [], level)
    ks_baby = host(ksa.keyswitch(prm, dev(ct), dev(baby[0].b), baby[0].seed, level, baby[0].galois))
    assert_equal(one_baby, ks_baby, "one baby step")
    one_giant = _run(prm, ct, _const_diag(oprm, level, [[0], [1]]), [], giant, level)
    ks_giant = host(ksa.keyswitch(prm, dev(ct), dev(giant[0].b), giant[0].seed, level, giant[0].galois))
    assert_equal(one_giant, ks_giant, "one giant step")
    prm.close()


def test_bsgs16_four_by_four():
    """N=2^16, L=24, dnum=4, K=6: 4 x 4 diagonals, baby X^(5^i), giant X^(5^(4j))."""
    w = ki.WORKLOADS["bsgs16"]
    n1, n2 = w.extra["n1"], w.extra["n2"]
    prm, oprm = params_pair(w.log2n, w.L, w.dnum, w.K, max_batch=8)  # the arena then fits 4 x 4 at L=24
    beta = len(oprm.digits(w.L))
    keys = [ks.Key(b=ki.uniform_key_b(w.index, k, beta, oprm.basis(w.L), oprm.N), seed=ki.key_seed(w.index, k),
                   level=w.L, galois=g) for k, g in enumerate(w.galois)]
    baby, giant = keys[: n1 - 1], keys[n1 - 1:]
    ct = ki.ciphertexts(w.index, oprm.q, oprm.N, 1)[0]
    diag = ki.uniform_diagonals(w.index, n2, n1, oprm.basis(w.L), oprm.N)
    out = _run(prm, ct, diag, baby, giant, w.L)
    assert_equal(out, bsgs.linear_transform(oprm, ct, diag, baby, giant, w.L), "bsgs16")
    again = _run(prm, ct, diag, baby, giant, w.L)
    assert_equal(again, out, "repeat")
    prm.close()


def _uniform_case(oprm, widx, level, baby_g, giant_g):
    kl = oprm.key_level(level)
    beta = len(oprm.digits(kl))
    keys = [ks.Key(b=ki.uniform_key_b(widx, k, beta, oprm.basis(kl), oprm.N), seed=ki.key_seed(widx, k),
                   level=kl, galois=g) for k, g in enumerate(list(baby_g) + list(giant_g))]
    ct = ki.ciphertexts(widx, oprm.q[:level], oprm.N, 1)[0]
    diag = ki.uniform_diagonals(widx, len(giant_g) + 1, len(baby_g) + 1, oprm.basis(level), oprm.N)
    return ct, diag, keys[: len(baby_g)], keys[len(baby_g):]


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes_match_oracle(seed):
    """Seeded random N=2^12 chains, levels and step counts with uniform keys and
    diagonals; Galois elements drawn with 1 and 2N - 1 among them, so that giant
    steps also run in natural order (every giant element 1) and mixed."""
    g = np.random.default_rng([11, seed])
    L = int(g.integers(1, 10))
    dnum = int(g.integers(-(-L // 8), min(L, 6) + 1))
    K = int(g.integers(1, 4))
    partition = int(g.integers(0, 2))
    level = int(g.integers(1, L + 1))
    n1, n2 = int(g.integers(1, 6)), int(g.integers(1, 6))
    n2N = 2 << 12
    pool = [1, n2N - 1, 5, 25, 3125]
    baby_g = [pool[int(i)] for i in g.integers(0, len(pool), n1 - 1)]
    giant_g = [1] * (n2 - 1) if seed % 3 == 0 else [pool[int(i)] for i in g.integers(0, len(pool), n2 - 1)]
    what = f"seed {seed}: L={L} dnum={dnum} K={K} partition={partition} level={level} baby={baby_g} giant={giant_g}"
    print(what, flush=True)
    prm, oprm = params_pair(12, L, dnum, K, partition=partition, max_batch=8, max_hoist=8)
    ct, diag, baby, giant = _uniform_case(oprm, 500 + seed, level, baby_g, giant_g)
    out = _run(prm, ct, diag, baby, giant, level)
    assert_equal(out, bsgs.linear_transform(oprm, ct, diag, baby, giant, level), what)
    prm.close()
