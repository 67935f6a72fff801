"""Bit-exact parity of the HIP path (through the C ABI) with the CPU oracle.

Everything here is integer arithmetic, so the bar is equality of every word.
Inputs are seeded synthetic draws from ks_inputs; keys come from the oracle's
key generation or are uniform b halves with a ChaCha seed (bit-exactness does
not depend on b being a real key). The oracle computes its own primes, which
must equal the library's. The steps (NTT, ModUp, ModDown, the ChaCha
expander) are compared here at every ring size; whole key switches at the
full sizes, every output item of them, are in test_gpu_fullsize.py.
"""

import shutil
import subprocess

import numpy as np
import pytest

import ks_inputs as ki
from oracle import chacha
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
    oprm = ks.Params(log2n, L, dnum, K, chacha_rounds=kw.get("chacha_rounds", 12), partition=kw.get("partition", 0))
    assert tuple(prm.primes) == oprm.primes
    assert tuple(prm.psi) == tuple(rns.find_psi(p, oprm.N) for p in oprm.primes)
    return prm, oprm


# ---------------------------------------------------------------------------
# NTT
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("log2n,L,dnum,K", [(12, 3, 1, 1), (16, 24, 4, 6), (17, 40, 5, 8)])
def test_ntt_and_intt_match_oracle(log2n, L, dnum, K):
    prm, oprm = params_pair(log2n, L, dnum, K)
    N = oprm.N
    primes = oprm.primes
    idx = list(range(len(primes)))[::-1]  # a non-trivial prime order
    x = ki.uniform_limbs(np.random.default_rng(log2n), [primes[i] for i in idx], N)
    t = dev(x)
    ksa.ntt(prm, t, idx)
    fw = host(t)
    for z in range(0, len(idx), max(1, len(idx) // 8)):
        assert_equal(fw[z], rns.ntt(x[z], primes[idx[z]]), f"ntt limb {z}")
    ksa.intt(prm, t, idx)
    assert_equal(host(t), x, "intt(ntt(x))")
    t2 = dev(x)
    ksa.intt(prm, t2, idx)
    back = host(t2)
    for z in range(0, len(idx), max(1, len(idx) // 8)):
        assert_equal(back[z], rns.intt(x[z], primes[idx[z]]), f"intt limb {z}")
    prm.close()


def test_ntt_many_polynomials():
    """count polynomials of nlimbs limbs in one call: limb z of each uses prime_idx[z]."""
    prm, oprm = params_pair(12, 3, 3, 2)
    idx = [4, 0, 2]
    primes = oprm.primes
    x = np.stack([ki.uniform_limbs(np.random.default_rng(90 + c), [primes[i] for i in idx], oprm.N)
                  for c in range(5)])
    t = dev(x)
    ksa.ntt(prm, t, idx)
    fw = host(t)
    for c in range(5):
        for z, pi in enumerate(idx):
            assert_equal(fw[c, z], rns.ntt(x[c, z], primes[pi]), f"poly {c} limb {z}")
    ksa.intt(prm, t, idx)
    assert_equal(host(t), x, "intt(ntt(x)) over 5 polynomials")
    prm.close()


def test_ntt_edge_values():
    prm, oprm = params_pair(16, 2, 1, 1)
    N, q = oprm.N, oprm.primes[0]
    cases = np.stack([np.zeros(N), np.full(N, q - 1), np.eye(1, N, 0)[0], np.eye(1, N, N - 1)[0]]).astype(np.uint64)
    t = dev(cases)
    ksa.ntt(prm, t, [0] * 4)
    out = host(t)
    for z in range(4):
        assert_equal(out[z], rns.ntt(cases[z], q), f"edge case {z}")
    prm.close()


# ---------------------------------------------------------------------------
# ChaCha expander
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("log2n,L,dnum,K", [(12, 3, 3, 1), (16, 24, 4, 6)])
def test_chacha_expand_matches_oracle(log2n, L, dnum, K):
    prm, oprm = params_pair(log2n, L, dnum, K)
    seed = bytes(range(7, 39))
    for level in (L, max(1, L // 2)):
        basis = oprm.basis(level)
        for d in range(len(oprm.digits(level))):
            for j in (0, level - 1, level, len(basis) - 1):
                g = host(ksa.chacha_expand(prm, seed, d, j, level))
                assert_equal(g, chacha.expand_uniform(seed, d, j, oprm.N, basis[j], 12), f"a[{d}][{j}] l={level}")
    prm.close()


@pytest.mark.skipif(shutil.which("openssl") is None, reason="openssl command line not available")
def test_chacha20_expand_matches_openssl():
    prm, oprm = params_pair(12, 3, 3, 1, chacha_rounds=20)
    seed = bytes(range(100, 132))
    N = oprm.N
    for d, j in ((0, 0), (2, 3)):
        r = oprm.basis(3)[j]
        iv = bytes(4) + (0).to_bytes(4, "little") + d.to_bytes(4, "little") + j.to_bytes(4, "little")
        res = subprocess.run(["openssl", "enc", "-chacha20", "-K", seed.hex(), "-iv", iv.hex()],
                             input=bytes(8 * N), stdout=subprocess.PIPE, check=True)
        ref = [int.from_bytes(res.stdout[8 * i: 8 * i + 8], "little") % r for i in range(N)]
        assert_equal(host(ksa.chacha_expand(prm, seed, d, j, 3)), ref, f"chacha20 a[{d}][{j}]")
    prm.close()


# ---------------------------------------------------------------------------
# ModUp and ModDown
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("log2n,L,dnum,K,levels", [
    (12, 3, 3, 1, (3, 2, 1)),
    (12, 7, 3, 2, (7, 5, 4, 1)),   # short last digit, one-prime digits
    (16, 24, 4, 6, (24, 13)),
])
def test_modup_matches_oracle(log2n, L, dnum, K, levels):
    prm, oprm = params_pair(log2n, L, dnum, K)
    for level in levels:
        c1 = ki.uniform_limbs(np.random.default_rng(level), oprm.q[:level], oprm.N)
        ext = host(ksa.modup(prm, dev(c1), level))
        assert_equal(ext, ks.modup(oprm, c1, level), f"modup level {level}")
    prm.close()


@pytest.mark.parametrize("log2n,L,dnum,K,levels", [
    (12, 3, 3, 1, (3, 1)),
    (12, 7, 3, 3, (7, 2)),
    (16, 24, 4, 6, (24, 9)),
])
def test_moddown_matches_oracle(log2n, L, dnum, K, levels):
    prm, oprm = params_pair(log2n, L, dnum, K)
    for level in levels:
        acc = ki.uniform_limbs(np.random.default_rng(100 + level), oprm.basis(level), oprm.N)
        out = host(ksa.moddown(prm, dev(acc), level))
        assert_equal(out, ks.moddown(oprm, acc, level), f"moddown level {level}")
    prm.close()


# ---------------------------------------------------------------------------
# whole key switch
# ---------------------------------------------------------------------------

def _real_keys(oprm, widx, level, galois_list, h):
    s = ki.ternary_secret(widx, oprm.N, h)
    keys, emax = [], 0
    for kidx, g in enumerate(galois_list):
        errs = ki.gaussian_errors(widx, kidx, len(oprm.digits(level)), oprm.N)
        emax = max(emax, int(np.abs(errs).max()))
        keys.append(ks.keygen(oprm, s, errs, ki.key_seed(widx, kidx), level, g))
    return s, keys, emax


def _uniform_keys(oprm, widx, level, galois_list):
    beta = len(oprm.digits(level))
    return [ks.Key(b=ki.uniform_key_b(widx, k, beta, oprm.basis(level), oprm.N), seed=ki.key_seed(widx, k),
                   level=level, galois=g) for k, g in enumerate(galois_list)]


def _decrypts(oprm, ct, out, s, galois, level, emax, h):
    e = ks.decryption_error(oprm, ct, out, s, galois, level)
    assert e is not None, "error residues differ between limbs"
    assert np.abs(e).max() <= ks.error_bound(oprm, level, emax, h)


def test_tiny_rotation_bit_exact_and_decrypts():
    w = ki.WORKLOADS["tiny"]
    prm, oprm = params_pair(w.log2n, w.L, w.dnum, w.K)
    s, (key,), emax = _real_keys(oprm, w.index, w.L, (5,), w.h)
    ct = ki.ciphertexts(w.index, oprm.q, oprm.N, 1)[0]
    out = host(ksa.keyswitch(prm, dev(ct), dev(key.b), key.seed, w.L, 5))
    assert_equal(out, ks.keyswitch(oprm, ct, key, w.L), "tiny key switch")
    _decrypts(oprm, ct, out, s, 5, w.L, emax, w.h)
    prm.close()


@pytest.mark.parametrize("level,galois", [(7, 1), (7, 8191), (5, 25), (4, 5), (1, 5), (1, 1)])
def test_small_ring_levels_and_partitions(level, galois):
    # K = 3 special primes: P is about as large as the biggest digit (3 primes),
    # which the decryption bound needs; digits at level 7 are 3, 3 and 1 primes.
    prm, oprm = params_pair(12, 7, 3, 3)
    s, (key,), emax = _real_keys(oprm, 20 + level, level, (galois,), 32)
    ct = ki.ciphertexts(20 + level, oprm.q[:level], oprm.N, 1)[0]
    out = host(ksa.keyswitch(prm, dev(ct), dev(key.b), key.seed, level, galois))
    assert_equal(out, ks.keyswitch(oprm, ct, key, level), f"level {level} galois {galois}")
    _decrypts(oprm, ct, out, s, galois, level, emax, 32)
    prm.close()


@pytest.mark.parametrize("level", [7, 5, 4, 2, 1])
def test_small_ring_top_level_partition(level):
    """Partition 1: one key generated at L = 7 serves every level (alpha = 3 fixed);
    batch of 2 under a rotation and the relinearisation key, regenerated and stored a."""
    prm, oprm = params_pair(12, 7, 3, 3, partition=1, max_batch=2, max_hoist=2)
    assert prm.key_shape(level) == (3, 10, 4096)
    s, keys, emax = _real_keys(oprm, 40, 7, (5, 1), 32)
    cts = ki.ciphertexts(40 + level, oprm.q[:level], oprm.N, 2)
    kb = [dev(k.b) for k in keys]
    out = host(ksa.keyswitch_ex(prm, dev(cts), kb, [k.galois for k in keys], level, seeds=[k.seed for k in keys]))
    for r, key in enumerate(keys):
        for b in range(2):
            ref = ks.keyswitch(oprm, cts[b], key, level)
            assert_equal(out[r, b], ref, f"level {level} key {r} item {b}")
        _decrypts(oprm, cts[1], out[r, 1], s, key.galois, level, emax, 32)
    stored = host(ksa.keyswitch_ex(prm, dev(cts), kb, [k.galois for k in keys], level,
                                   evk_a=[dev(ks.key_a(oprm, k)) for k in keys]))
    assert_equal(stored, out, f"level {level} stored vs regenerated")
    single = host(ksa.keyswitch(prm, dev(cts[0]), kb[0], keys[0].seed, level, 5))
    assert_equal(single, out[0, 0], f"level {level} pc_keyswitch")
    prm.close()


def _keygen_inputs(oprm, widx, level, s):
    """Residues of the secret and of each digit's errors over the key basis (test-side marshalling)."""
    basis = oprm.basis(level)
    errs = ki.gaussian_errors(widx, 0, len(oprm.digits(level)), oprm.N)
    s_coef = np.stack([rns.to_residues(s, r) for r in basis])
    e_coef = np.stack([np.stack([rns.to_residues(errs[d], r) for r in basis]) for d in range(len(errs))])
    return errs, s_coef, e_coef


@pytest.mark.parametrize("log2n,L,dnum,K,level,galois,partition,h", [
    (12, 3, 3, 1, 3, 5, 0, 64),        # the tiny rotation key
    (12, 7, 3, 3, 5, 25, 0, 32),       # a rotation key below the top level
    (12, 7, 3, 3, 7, 1, 1, 32),        # the top-level key of partition 1 (relinearisation)
    (16, 24, 4, 6, 24, 1, 0, 192),     # the full-size relinearisation key
])
def test_keygen_matches_oracle(log2n, L, dnum, K, level, galois, partition, h):
    """pc_keygen against the oracle's key generation, bit for bit; the GPU key then
    drives a GPU key switch that decrypts within the bound."""
    prm, oprm = params_pair(log2n, L, dnum, K, partition=partition)
    widx = 50 + level
    s = ki.ternary_secret(widx, oprm.N, h)
    errs, s_coef, e_coef = _keygen_inputs(oprm, widx, level, s)
    seed = ki.key_seed(widx, 3)
    key = ks.keygen(oprm, s, errs, seed, level, galois)
    b = host(ksa.keygen(prm, seed, level, galois, dev(s_coef), dev(e_coef)))
    assert_equal(b, key.b, f"key b, level {level} galois {galois}")
    ct_level = level if partition == 0 else max(1, level - 2)
    ct = ki.ciphertexts(widx, oprm.q[:ct_level], oprm.N, 1)[0]
    out = host(ksa.keyswitch(prm, dev(ct), dev(b), seed, ct_level, galois))
    assert_equal(out, ks.keyswitch(oprm, ct, key, ct_level), "key switch with the GPU key")
    _decrypts(oprm, ct, out, s, galois, ct_level, int(np.abs(errs).max()), h)
    prm.close()


def test_caller_workspace_matches_arena():
    prm, oprm = params_pair(12, 7, 3, 2, max_batch=3, max_hoist=2)
    keys = _uniform_keys(oprm, 77, 7, (5, 1))
    cts = ki.ciphertexts(77, oprm.q, oprm.N, 3)
    kbs = [dev(k.b) for k in keys]
    seeds = [k.seed for k in keys]
    a = host(ksa.keyswitch_ex(prm, dev(cts), kbs, [5, 1], 7, seeds=seeds))
    ws = torch.empty(prm.workspace_bytes(7) // 4, dtype=torch.int32, device="cuda:0")
    b = host(ksa.keyswitch_ex(prm, dev(cts), kbs, [5, 1], 7, seeds=seeds, workspace=ws))
    assert_equal(a, b, "caller workspace")
    ref = ks.keyswitch_hoisted(oprm, cts[2], keys, 7)
    assert_equal(a[:, 2], ref, "3-item batch, 2 keys")
    # one ciphertext: the segment layout, also read by the key with g = 1; a regenerated and stored
    one = host(ksa.keyswitch_ex(prm, dev(cts[2:3]), kbs, [5, 1], 7, seeds=seeds))
    assert_equal(one[:, 0], ref, "1 item, 2 keys")
    one_stored = host(ksa.keyswitch_ex(prm, dev(cts[2:3]), kbs, [5, 1], 7, evk_a=[dev(ks.key_a(oprm, k)) for k in keys]))
    assert_equal(one_stored, one, "1 item, 2 keys, stored a")
    small = torch.empty(16, dtype=torch.int32, device="cuda:0")
    with pytest.raises(ksa.PcError):
        ksa.keyswitch_ex(prm, dev(cts), kbs, [5, 1], 7, seeds=seeds, workspace=small)
    prm.close()


def test_rejected_arguments_on_gpu():
    prm, oprm = params_pair(12, 3, 3, 1)
    ct = dev(np.zeros((2, 3, oprm.N), dtype=np.uint32))
    b = dev(np.zeros((3, 4, oprm.N), dtype=np.uint32))
    with pytest.raises(ksa.PcError) as e:
        ksa.keyswitch(prm, ct, b, bytes(32), 3, 4)
    assert e.value.code == ksa.PC_EINVAL
    with pytest.raises(ValueError):
        ksa.keyswitch(prm, ct[:, :2].contiguous(), b, bytes(32), 3, 5)
    prm.close()


def test_allocation_failure_reports_enomem():
    """An arena too large for the device fails creation with PC_ENOMEM, and the
    library keeps working afterwards (the failure is not left for a later launch)."""
    with pytest.raises(ksa.PcError) as e:
        ksa.Params(16, 24, 4, 6, max_batch=1 << 20, device=0)
    assert e.value.code == ksa.PC_ENOMEM
    w = ki.WORKLOADS["tiny"]
    prm, oprm = params_pair(w.log2n, w.L, w.dnum, w.K)
    s, (key,), _ = _real_keys(oprm, w.index, w.L, (5,), w.h)
    ct = ki.ciphertexts(w.index, oprm.q, oprm.N, 1)[0]
    out = host(ksa.keyswitch(prm, dev(ct), dev(key.b), key.seed, w.L, 5))
    assert_equal(out, ks.keyswitch(oprm, ct, key, w.L), "key switch after a failed creation")
    prm.close()
