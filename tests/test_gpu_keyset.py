"""Key switches drawn from a key bundle (packed: b halves plus seeds; full: the a
halves stored too) against the oracle.

A bundle holds every key in one device allocation. Keys enter it by copy
(pc_keyset_set) or by generation in place (pc_keyset_keygen); key switches read
them by index (pc_keyswitch_keyset). Outputs are compared word for word with
the oracle's key switch (small ring) or with the stored digests of the oracle's
outputs (the 16 hoisted rotation keys at N = 2^16).
"""

import os
import sys

import numpy as np
import pytest

import ks_inputs as ki
from oracle import keyswitch as ks
from oracle import rns

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden"))
import cases  # noqa: E402

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


@pytest.mark.parametrize("full", [False, True])
def test_generated_bundle_small_ring(full):
    """N = 2^12, L = 7, dnum = 3, K = 3: three keys (X^5, X^25, relinearisation) generated
    into the bundle on the GPU from the oracle's secret and errors; a batch of two
    ciphertexts under all three keys, and under two of them in another order."""
    L, level = 7, 7
    prm = ksa.Params(12, L, 3, 3, device=0, max_batch=2, max_hoist=3)
    oprm = ks.Params(12, L, 3, 3)
    galois = [5, 25, 1]
    s = ki.ternary_secret(70, oprm.N, 32)
    basis = oprm.basis(level)
    beta = len(oprm.digits(level))
    keys, emax = [], 0
    with ksa.KeySet(prm, level, galois, full=full) as bundle:
        assert bundle.key_bytes() == beta * len(basis) * oprm.N * 4
        assert bundle.device_bytes() == (2 if full else 1) * 3 * bundle.key_bytes()
        s_coef = dev(np.stack([rns.to_residues(s, r) for r in basis]))
        for k, g in enumerate(galois):
            errs = ki.gaussian_errors(70, k, beta, oprm.N)
            emax = max(emax, int(np.abs(errs).max()))
            e_coef = dev(np.stack([np.stack([rns.to_residues(errs[d], r) for r in basis]) for d in range(beta)]))
            seed = ki.key_seed(70, k)
            bundle.keygen(k, seed, s_coef, e_coef)
            keys.append(ks.keygen(oprm, s, errs, seed, level, g))
        cts = ki.ciphertexts(71, oprm.q[:level], oprm.N, 2)
        out = host(ksa.keyswitch_keyset(prm, bundle, dev(cts), [0, 1, 2], level))
        for b in range(2):
            want = ks.keyswitch_hoisted(oprm, cts[b], keys, level)
            for r in range(3):
                assert np.array_equal(out[r, b].astype(np.uint64), want[r]), (full, r, b)
                e = ks.decryption_error(oprm, cts[b], out[r, b], s, galois[r], level)
                assert e is not None and np.abs(e).max() <= ks.error_bound(oprm, level, emax, 32)
        sub = host(ksa.keyswitch_keyset(prm, bundle, dev(cts), [2, 0], level))
        assert np.array_equal(sub[0], out[2]) and np.array_equal(sub[1], out[0])
        # the relinearisation key alone takes the fused ModUp/inner-product tile
        one = host(ksa.keyswitch_keyset(prm, bundle, dev(cts), [2], level))
        assert np.array_equal(one[0], out[2]), full
        with pytest.raises(ksa.PcError):
            ksa.keyswitch_keyset(prm, bundle, dev(cts), [3], level)
    prm.close()


@pytest.mark.parametrize("full", [False, True])
def test_hoisted16_from_bundle_every_key(full):
    """The 16 rotation keys of the hoisted workload copied into a bundle; one N = 2^16
    ciphertext under all 16, every output against the oracle's digests."""
    c = cases.case_n16_hoist16()
    doc = cases.load_digests()
    assert doc["sources_hash"] == cases.sources_hash()
    want = doc["cases"][c.name]["digests"]
    prm = ksa.Params(c.prm.log2n, c.prm.L, c.prm.dnum, c.prm.K, device=0, max_hoist=16)
    with ksa.KeySet(prm, c.level, [k.galois for k in c.keys], full=full) as bundle:
        for r, k in enumerate(c.keys):
            bundle.set(r, dev(k.b), k.seed)
        out = host(ksa.keyswitch_keyset(prm, bundle, dev(c.cts), list(range(16)), c.level))
        for r in range(16):
            assert cases.digest(out[r, 0]) == want[r], f"key {r} (full={full})"
        pick = [11, 2, 7]
        sub = host(ksa.keyswitch_keyset(prm, bundle, dev(c.cts), pick, c.level))
        for n, r in enumerate(pick):
            assert cases.digest(sub[n, 0]) == want[r], f"selected key {r}"
    prm.close()


@pytest.mark.parametrize("full", [False, True])
def test_relinearisation_key_from_bundle_every_item(full):
    """The headline's relinearisation key (N = 2^16, L = 24) in a bundle, drawn alone
    for the batch of 8 (the fused tile with the bundle's b half and seed, or with its
    stored a half); every item against the oracle's digests."""
    c = cases.case_n16_relin_k8()
    doc = cases.load_digests()
    assert doc["sources_hash"] == cases.sources_hash()
    want = doc["cases"][c.name]["digests"]
    prm = ksa.Params(c.prm.log2n, c.prm.L, c.prm.dnum, c.prm.K, device=0, max_batch=8)
    key = c.keys[0]
    with ksa.KeySet(prm, c.level, [key.galois], full=full) as bundle:
        bundle.set(0, dev(key.b), key.seed)
        out = host(ksa.keyswitch_keyset(prm, bundle, dev(c.cts), [0], c.level))
        for b in range(c.batch):
            assert cases.digest(out[0, b]) == want[b], f"item {b} (full={full})"
    prm.close()
