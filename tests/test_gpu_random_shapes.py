"""Bit-exact parity of the key switch over seeded random small shapes.

The fixed cases elsewhere follow the workloads; these draw, at N = 2^12, the
chain (L, dnum, K), the digit partition, the ChaCha rounds, the ciphertext
level, the batch, the number of keys and their Galois elements (1, 2N - 1 and
random odd elements mixed), and whether the a halves are regenerated or
stored, and compare every output word of pc_keyswitch_ex with the oracle's
hoisted key switch. Batches of one take the segment-layout gathers, larger
batches the natural-order ones. Keys are uniform b halves with a ChaCha seed:
bit-exactness does not depend on b being a real key.
"""

import numpy as np
import pytest

import ks_inputs as ki
from oracle import keyswitch as ks

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ksa = pytest.importorskip("key_switching_amd")

LOG2N = 12
CASES = 96


def _shape(seed):
    g = np.random.default_rng([7, seed])
    L = int(g.integers(1, 13))
    dnum = int(g.integers(-(-L // 8), min(L, 6) + 1))  # at most 8 primes per digit and 6 digits
    K = int(g.integers(1, 5))
    partition = int(g.integers(0, 2))
    rounds = (12, 20)[int(g.integers(0, 2))]
    level = int(g.integers(1, L + 1))
    batch = (1, 1, 2, 3)[int(g.integers(0, 4))]
    nkeys = int(g.integers(1, 4))
    n2 = 2 << LOG2N
    pool = [1, n2 - 1] + [int(2 * g.integers(1, n2 // 2) + 1) % n2 for _ in range(4)]
    galois = [pool[int(i)] for i in g.integers(0, len(pool), nkeys)]
    stored = bool(g.integers(0, 2))
    return L, dnum, K, partition, rounds, level, batch, galois, stored


@pytest.mark.parametrize("seed", range(CASES))
def test_random_shape_matches_oracle(seed):
    L, dnum, K, partition, rounds, level, batch, galois, stored = _shape(seed)
    what = (f"seed {seed}: L={L} dnum={dnum} K={K} partition={partition} rounds={rounds} level={level} "
            f"batch={batch} galois={galois} stored={stored}")
    print(what, flush=True)
    prm = ksa.Params(LOG2N, L, dnum, K, device=0, partition=partition, chacha_rounds=rounds, max_batch=batch,
                     max_hoist=len(galois))
    oprm = ks.Params(LOG2N, L, dnum, K, chacha_rounds=rounds, partition=partition)
    assert tuple(prm.primes) == oprm.primes
    kl = oprm.key_level(level)
    beta = len(oprm.digits(kl))
    keys = [ks.Key(b=ki.uniform_key_b(300 + seed, k, beta, oprm.basis(kl), oprm.N), seed=ki.key_seed(300 + seed, k),
                   level=kl, galois=gal) for k, gal in enumerate(galois)]
    cts = ki.ciphertexts(300 + seed, oprm.q[:level], oprm.N, batch)
    kb = [ksa.to_device(k.b, 0) for k in keys]
    if stored:
        out = ksa.keyswitch_ex(prm, ksa.to_device(cts, 0), kb, galois, level,
                               evk_a=[ksa.to_device(ks.key_a(oprm, k), 0) for k in keys])
    else:
        out = ksa.keyswitch_ex(prm, ksa.to_device(cts, 0), kb, galois, level, seeds=[k.seed for k in keys])
    torch.cuda.synchronize()
    got = ksa.to_host(out).astype(np.uint64)
    for b in range(batch):
        want = ks.keyswitch_hoisted(oprm, cts[b], keys, level)
        for r in range(len(keys)):
            bad = np.flatnonzero(got[r, b].reshape(-1) != np.asarray(want[r], dtype=np.uint64).reshape(-1))
            assert bad.size == 0, f"{what}: key {r} item {b}: {bad.size} words differ, first at {bad[0]}"
    prm.close()


@pytest.mark.parametrize("L,dnum", [(10, 5), (12, 6)])
@pytest.mark.parametrize("batch", [1, 2])
@pytest.mark.parametrize("stored", [False, True])
def test_five_and_six_digits(L, dnum, batch, stored):
    """The largest digit counts in both gather layouts (one ciphertext: segment layout;
    two: natural order), with a rotation and the conjugation key, a regenerated or stored."""
    K, level, galois = 3, L, [5, (2 << LOG2N) - 1]
    prm = ksa.Params(LOG2N, L, dnum, K, device=0, max_batch=batch, max_hoist=2)
    oprm = ks.Params(LOG2N, L, dnum, K)
    assert len(oprm.digits(level)) == dnum
    widx = 400 + 10 * L + batch
    keys = [ks.Key(b=ki.uniform_key_b(widx, k, dnum, oprm.basis(level), oprm.N), seed=ki.key_seed(widx, k),
                   level=level, galois=g) for k, g in enumerate(galois)]
    cts = ki.ciphertexts(widx, oprm.q[:level], oprm.N, batch)
    kb = [ksa.to_device(k.b, 0) for k in keys]
    if stored:
        out = ksa.keyswitch_ex(prm, ksa.to_device(cts, 0), kb, galois, level,
                               evk_a=[ksa.to_device(ks.key_a(oprm, k), 0) for k in keys])
    else:
        out = ksa.keyswitch_ex(prm, ksa.to_device(cts, 0), kb, galois, level, seeds=[k.seed for k in keys])
    torch.cuda.synchronize()
    got = ksa.to_host(out).astype(np.uint64)
    for b in range(batch):
        want = ks.keyswitch_hoisted(oprm, cts[b], keys, level)
        for r in range(len(keys)):
            bad = np.flatnonzero(got[r, b].reshape(-1) != np.asarray(want[r], dtype=np.uint64).reshape(-1))
            assert bad.size == 0, f"beta {dnum} batch {batch} stored {stored}: key {r} item {b}: {bad.size} differ"
    prm.close()


def test_lower_level_with_more_digits():
    """Regression: with L = 6 and dnum = 5, level 5 has five digits against the
    top level's three, so its workspace is larger; the arena must cover it
    (seed 495 of the same draw: level 5, one ciphertext, two keys, stored a)."""
    assert _shape(495)[:3] == (6, 5, 2) and _shape(495)[5] == 5
    test_random_shape_matches_oracle(495)


def _shape8(seed):
    g = np.random.default_rng([8, seed])
    L = int(g.integers(2, 13))
    dnum = int(g.integers(-(-L // 8), min(L, 6) + 1))
    K = int(g.integers(1, 5))
    level = int(g.integers(1, L + 1))
    nkeys = int(g.integers(1, 3))
    n2 = 2 << LOG2N
    pool = [1, n2 - 1, 5, int(2 * g.integers(1, n2 // 2) + 1) % n2]
    galois = [pool[int(i)] for i in g.integers(0, len(pool), nkeys)]
    return L, dnum, K, level, galois, bool(seed % 2)


@pytest.mark.parametrize("seed", range(16))
def test_batch8_random_shapes_match_oracle(seed):
    """Batches of exactly 8 ciphertexts (the batch size the inner-product kernels are
    specialised for) over random chains, levels, digit counts and keys, the a half
    regenerated (even seeds) or stored (odd seeds); every output word."""
    L, dnum, K, level, galois, stored = _shape8(seed)
    what = f"seed {seed}: L={L} dnum={dnum} K={K} level={level} galois={galois} stored={stored}"
    print(what, flush=True)
    prm = ksa.Params(LOG2N, L, dnum, K, device=0, max_batch=8, max_hoist=len(galois))
    oprm = ks.Params(LOG2N, L, dnum, K)
    assert tuple(prm.primes) == oprm.primes
    beta = len(oprm.digits(level))
    keys = [ks.Key(b=ki.uniform_key_b(600 + seed, k, beta, oprm.basis(level), oprm.N),
                   seed=ki.key_seed(600 + seed, k), level=level, galois=gal) for k, gal in enumerate(galois)]
    cts = ki.ciphertexts(600 + seed, oprm.q[:level], oprm.N, 8)
    kb = [ksa.to_device(k.b, 0) for k in keys]
    if stored:
        out = ksa.keyswitch_ex(prm, ksa.to_device(cts, 0), kb, galois, level,
                               evk_a=[ksa.to_device(ks.key_a(oprm, k), 0) for k in keys])
    else:
        out = ksa.keyswitch_ex(prm, ksa.to_device(cts, 0), kb, galois, level, seeds=[k.seed for k in keys])
    torch.cuda.synchronize()
    got = ksa.to_host(out).astype(np.uint64)
    for b in range(8):
        want = ks.keyswitch_hoisted(oprm, cts[b], keys, level)
        for r in range(len(keys)):
            bad = np.flatnonzero(got[r, b].reshape(-1) != np.asarray(want[r], dtype=np.uint64).reshape(-1))
            assert bad.size == 0, f"{what}: key {r} item {b}: {bad.size} words differ, first at {bad[0]}"
    prm.close()
