"""Bit-exact parity of the GPU homomorphic multiplication (pc_tensor,
pc_rescale, pc_hmult through the C ABI) with the oracle's tensor product,
rounded rescale and relinearisation.

Inputs are seeded synthetic ciphertexts from ks_inputs; relinearisation keys
come from the oracle's key generation (small rings) or are uniform b halves with
a ChaCha seed (the headline ring: bit-exactness does not depend on b being a
real key).
"""

import numpy as np
import pytest

import ks_inputs as ki
from oracle import hmult as hm
from oracle import keyswitch as ks
from oracle import rns

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


def _pairs(widx, oprm, level, batch):
    cts = ki.ciphertexts(widx, oprm.q[:level], oprm.N, 2 * batch)
    return cts[:batch], cts[batch:]


@pytest.mark.parametrize("log2n,L,dnum,K,level,batch", [
    (12, 7, 3, 3, 7, 2), (12, 7, 3, 3, 1, 1), (16, 24, 4, 6, 24, 8), (16, 24, 4, 6, 13, 3)])
def test_tensor_matches_oracle(log2n, L, dnum, K, level, batch):
    prm, oprm = params_pair(log2n, L, dnum, K, max_batch=8)
    a, b = _pairs(80 + level, oprm, level, batch)
    d = host(ksa.tensor(prm, dev(a), dev(b), level))
    for z in range(batch):
        assert_equal(d[z], hm.tensor(oprm, a[z], b[z], level), f"tensor level {level} pair {z}")
    prm.close()


def _edge_last_limb(oprm, ct, level):
    """Put the rounding boundaries into the dropped limb's coefficients: 0, 1,
    (q-1)/2 (largest kept positive), (q+1)/2 (first negative), q-1, q-2, then random."""
    ql = oprm.q[level - 1]
    coef = rns.intt(ct[0, level - 1], ql).astype(np.uint64)
    edges = np.array([0, 1, (ql - 1) // 2, (ql + 1) // 2, ql - 1, ql - 2], dtype=np.uint64)
    coef[: edges.size * 8] = np.tile(edges, 8)
    ct = ct.copy()
    ct[0, level - 1] = rns.ntt(coef, ql)
    return ct


@pytest.mark.parametrize("log2n,L,dnum,K,level,batch", [
    (12, 7, 3, 3, 7, 2), (12, 7, 3, 3, 2, 1), (12, 3, 3, 1, 3, 1), (16, 24, 4, 6, 24, 2), (16, 24, 4, 6, 9, 1)])
def test_rescale_matches_oracle(log2n, L, dnum, K, level, batch):
    prm, oprm = params_pair(log2n, L, dnum, K, max_batch=8)
    cts = ki.ciphertexts(90 + level, oprm.q[:level], oprm.N, batch)
    cts[0] = _edge_last_limb(oprm, cts[0], level)
    out = host(ksa.rescale(prm, dev(cts), level))
    for z in range(batch):
        assert_equal(out[z], hm.rescale(oprm, cts[z], level), f"rescale level {level} item {z}")
    prm.close()


@pytest.mark.parametrize("level,partition", [(7, 0), (4, 0), (2, 0), (7, 1), (3, 1), (2, 1)])
def test_small_ring_hmult_matches_oracle(level, partition):
    """N=2^12, L=7, dnum=3, K=3 with a real key of s^2 (at the key level the partition asks for)."""
    prm, oprm = params_pair(12, 7, 3, 3, partition=partition, max_batch=3)
    kl = oprm.key_level(level)
    s = ki.ternary_secret(100 + level, oprm.N, 32)
    errs = ki.gaussian_errors(100 + level, 0, len(oprm.digits(kl)), oprm.N)
    key = ks.keygen(oprm, s, errs, ki.key_seed(100 + level, 0), kl, 1)
    a, b = _pairs(100 + level, oprm, level, 3)
    out = host(ksa.hmult(prm, dev(a), dev(b), dev(key.b), key.seed, level))
    for z in range(3):
        assert_equal(out[z], hm.hmult(oprm, a[z], b[z], key, level), f"hmult level {level} pair {z}")
    # one pair alone gives the same bits as inside the batch
    one = host(ksa.hmult(prm, dev(a[1]), dev(b[1]), dev(key.b), key.seed, level))
    assert_equal(one[0], out[1], "batch of one vs batch of three")
    prm.close()


def test_headline_n16_hmult_batch8():
    """N=2^16, L=24, dnum=4, K=6: eight products at the top level (one key of s^2)."""
    w = ki.WORKLOADS["n16"]
    prm, oprm = params_pair(w.log2n, w.L, w.dnum, w.K, max_batch=8)
    (key,) = [ks.Key(b=ki.uniform_key_b(w.index, 0, len(oprm.digits(w.L)), oprm.basis(w.L), oprm.N),
                     seed=ki.key_seed(w.index, 0), level=w.L, galois=1)]
    a, b = _pairs(w.index + 7, oprm, w.L, 8)
    kb = dev(key.b)
    out = host(ksa.hmult(prm, dev(a), dev(b), kb, key.seed, w.L))
    assert out.shape == (8, 2, w.L - 1, oprm.N)
    for z in (0, 6):
        assert_equal(out[z], hm.hmult(oprm, a[z], b[z], key, w.L), f"n16 hmult pair {z}")
    again = host(ksa.hmult(prm, dev(a), dev(b), kb, key.seed, w.L))
    assert_equal(again, out, "repeat")
    prm.close()


def test_n17_hmult():
    """N=2^17, L=40, dnum=5, K=8: two products at the top level, rescaled to L=39."""
    w = ki.WORKLOADS["n17"]
    prm, oprm = params_pair(w.log2n, w.L, w.dnum, w.K, max_batch=2)
    key = ks.Key(b=ki.uniform_key_b(w.index, 0, len(oprm.digits(w.L)), oprm.basis(w.L), oprm.N),
                 seed=ki.key_seed(w.index, 0), level=w.L, galois=1)
    a, b = _pairs(w.index + 9, oprm, w.L, 2)
    out = host(ksa.hmult(prm, dev(a), dev(b), dev(key.b), key.seed, w.L))
    assert out.shape == (2, 2, w.L - 1, oprm.N)
    assert_equal(out[1], hm.hmult(oprm, a[1], b[1], key, w.L), "n17 hmult pair 1")
    prm.close()


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes_match_oracle(seed):
    """Seeded random N=2^12 chains, partitions, levels (>= 2, so that the rescale
    keeps a limb) and batches, with a uniform key b half and its ChaCha seed."""
    g = np.random.default_rng([13, seed])
    L = int(g.integers(2, 11))
    dnum = int(g.integers(-(-L // 8), min(L, 6) + 1))
    K = int(g.integers(1, 4))
    partition = int(g.integers(0, 2))
    level = int(g.integers(2, L + 1))
    batch = int(g.integers(1, 4))
    what = f"seed {seed}: L={L} dnum={dnum} K={K} partition={partition} level={level} batch={batch}"
    print(what, flush=True)
    prm, oprm = params_pair(12, L, dnum, K, partition=partition, max_batch=batch)
    kl = oprm.key_level(level)
    key = ks.Key(b=ki.uniform_key_b(600 + seed, 0, len(oprm.digits(kl)), oprm.basis(kl), oprm.N),
                 seed=ki.key_seed(600 + seed, 0), level=kl, galois=1)
    a, b = _pairs(600 + seed, oprm, level, batch)
    out = host(ksa.hmult(prm, dev(a), dev(b), dev(key.b), key.seed, level))
    for z in range(batch):
        assert_equal(out[z], hm.hmult(oprm, a[z], b[z], key, level), f"{what} pair {z}")
    prm.close()
