"""Key switches at the library's limits, bit-exact with the oracle (N = 2^12).

The limits are those pc_params_create and the launches accept: 32 keys in one
launch (the most a launch carries in its arguments), 8 special primes, 8
primes per digit and 6 digits, and a long chain (L + K = 56 limbs). Keys are
uniform b halves with a ChaCha seed (bit-exactness does not depend on b being
a real key); every output word is compared with the oracle's hoisted key
switch.
"""

import numpy as np
import pytest

import ks_inputs as ki
from oracle import keyswitch as ks

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ksa = pytest.importorskip("key_switching_amd")

LOG2N = 12


def _check(tag, L, dnum, K, level, batch, galois, stored=False):
    what = f"{tag}: L={L} dnum={dnum} K={K} level={level} batch={batch} keys={len(galois)} stored={stored}"
    print(what, flush=True)
    prm = ksa.Params(LOG2N, L, dnum, K, device=0, max_batch=batch, max_hoist=len(galois))
    oprm = ks.Params(LOG2N, L, dnum, K)
    assert tuple(prm.primes) == oprm.primes
    beta = len(oprm.digits(level))
    keys = [ks.Key(b=ki.uniform_key_b(900 + L, k, beta, oprm.basis(level), oprm.N), seed=ki.key_seed(900 + L, k),
                   level=level, galois=g) for k, g in enumerate(galois)]
    cts = ki.ciphertexts(900 + L, oprm.q[:level], oprm.N, batch)
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


@pytest.mark.parametrize("batch", [1, 2])
def test_thirty_two_keys_in_one_launch(batch):
    """The most keys a launch takes: relinearisation, conjugation and 30 rotations."""
    n2 = 2 << LOG2N
    galois = [1, n2 - 1] + [pow(5, r, n2) for r in range(1, 31)]
    _check("32 keys", 6, 3, 2, 6, batch, galois)


@pytest.mark.parametrize("stored", [False, True])
def test_eight_special_primes_and_eight_primes_per_digit(stored):
    _check("K=8, alpha=8", 16, 2, 8, 16, 2, [1, 5], stored)


@pytest.mark.parametrize("level", [48, 47, 2])
def test_long_chain(level):
    """L = 48, dnum = 6 (alpha = 8, six digits at the top), K = 8: 56 limbs."""
    _check("long chain", 48, 6, 8, level, 1, [3])
