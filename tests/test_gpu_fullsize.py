"""Every output item of the full-size workloads against the oracle.

The oracle's outputs for these cases are stored as one SHA-256 digest per
(key, ciphertext) item in tests/golden/digests_full.json, written by
tests/golden/make_digests.py from oracle/ alone; tests/golden/cases.py holds
the input recipe both sides use. Each test rebuilds the inputs, runs the
library through the C ABI in the configurations the benchmark times (batches
of 8 with a regenerated or stored a half, single ciphertexts, hoisted keys,
three streams with caller workspaces) and compares the digest of every output
item. On a mismatch the oracle is run for that item and the first differing
word is reported.
"""

import os
import sys

import numpy as np
import pytest

import ks_inputs as ki
from oracle import keyswitch as ks

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


@pytest.fixture(scope="module")
def digests():
    doc = cases.load_digests()
    assert doc["sources_hash"] == cases.sources_hash(), "stale digests: run tests/golden/make_digests.py"
    return doc["cases"]


def dev(a):
    return ksa.to_device(a, 0)


def host(t):
    torch.cuda.synchronize()
    return ksa.to_host(t)


def check_items(c, got, want, label, index=None, oracle_item=None):
    """Compare the digest of every item of got [R][B][2][l][N] (or a list of
    [2][l][N] arrays with their digest indices) with the stored ones."""
    bad = []
    for idx, arr in (index if index is not None else
                     [(r * got.shape[1] + b, got[r, b]) for r in range(got.shape[0]) for b in range(got.shape[1])]):
        if cases.digest(arr) != want[idx]:
            bad.append((idx, arr))
    if bad:
        idx, arr = bad[0]
        detail = ""
        if oracle_item is not None:
            ref = np.asarray(oracle_item(idx), dtype=np.uint64).reshape(-1)
            diff = np.flatnonzero(arr.astype(np.uint64).reshape(-1) != ref)
            detail = f"; item {idx}: {diff.size} words differ from the oracle, first at flat index {diff[:1]}"
        pytest.fail(f"{label}: {len(bad)} item(s) differ from the oracle's digests, first index {idx}{detail}")


def params_for(c, **kw):
    prm = ksa.Params(c.prm.log2n, c.prm.L, c.prm.dnum, c.prm.K, device=0, **kw)
    assert tuple(prm.primes) == c.prm.primes
    return prm


def run_case(prm, c, batch_items=None, single=False, stored=None, out=None, workspace=None):
    """GPU outputs [R][B][2][l][N] of case c (all keys in one call, or one call per
    ciphertext with single=True)."""
    stored = c.stored if stored is None else stored
    kb = [dev(k.b) for k in c.keys]
    galois = [k.galois for k in c.keys]
    ka = [dev(ks.key_a(c.prm, k)) for k in c.keys] if stored else None
    seeds = None if stored else [k.seed for k in c.keys]
    if single:
        res = [ksa.keyswitch_ex(prm, dev(c.cts[b:b + 1]), kb, galois, c.level, seeds=seeds, evk_a=ka)
               for b in range(c.batch)]
        return np.concatenate([host(r) for r in res], axis=1)
    return host(ksa.keyswitch_ex(prm, dev(c.cts), kb, galois, c.level, seeds=seeds, evk_a=ka, out=out,
                                 workspace=workspace))


def oracle_of(c):
    def item(idx):
        r, b = divmod(idx, c.batch)
        return ks.keyswitch(c.prm, c.cts[b], c.keys[r], c.level)
    return item


def test_n16_relinearisation_batch8_every_item(digests):
    """Headline workload: all 8 ciphertexts, batch call with the a half regenerated and
    with it stored, and each ciphertext alone (the k = 1 path)."""
    c = cases.case_n16_relin_k8()
    want = digests[c.name]["digests"]
    prm = params_for(c, max_batch=8)
    check_items(c, run_case(prm, c), want, "k=8 regenerated a", oracle_item=oracle_of(c))
    check_items(c, run_case(prm, c, stored=True), want, "k=8 stored a", oracle_item=oracle_of(c))
    check_items(c, run_case(prm, c, single=True), want, "k=1 regenerated a", oracle_item=oracle_of(c))
    check_items(c, run_case(prm, c, single=True, stored=True), want, "k=1 stored a", oracle_item=oracle_of(c))
    prm.close()


def test_n16_three_streams_every_item(digests):
    """The benchmark's launch configuration: batches of 8 dealt to three streams, each
    call with its own workspace; every item of every call against the digests."""
    c = cases.case_n16_relin_k8()
    want = digests[c.name]["digests"]
    prm = params_for(c, max_batch=8)
    kb = dev(c.keys[0].b)
    ct = dev(c.cts)
    streams = [torch.cuda.Stream() for _ in range(3)]
    ws = [torch.empty(prm.workspace_bytes(c.level) // 4, dtype=torch.int32, device="cuda:0") for _ in range(3)]
    outs = [torch.empty((1, 8, 2, c.level, c.prm.N), dtype=torch.int32, device="cuda:0") for _ in range(6)]
    torch.cuda.synchronize()
    for i in range(6):
        with torch.cuda.stream(streams[i % 3]):
            ksa.keyswitch_ex(prm, ct, [kb], [1], c.level, seeds=[c.keys[0].seed], out=outs[i], workspace=ws[i % 3])
    torch.cuda.synchronize()
    for i in range(6):
        check_items(c, host(outs[i]), want, f"three streams, call {i}")
    prm.close()


def test_n16_hoisted_sixteen_keys_every_key(digests):
    c = cases.case_n16_hoist16()
    want = digests[c.name]["digests"]
    prm = params_for(c, max_hoist=16)
    check_items(c, run_case(prm, c), want, "16 hoisted keys", oracle_item=oracle_of(c))
    # each key on its own (one key per call)
    kb = [dev(k.b) for k in c.keys]
    ct = dev(c.cts[0])
    got = [(r, host(ksa.keyswitch(prm, ct, kb[r], k.seed, c.level, k.galois))) for r, k in enumerate(c.keys)]
    check_items(c, None, want, "single-key calls", index=got)
    prm.close()


@pytest.mark.parametrize("level", cases.LEVELS)
def test_n16_level_sweep_every_item(digests, level):
    """8 ciphertexts x 2 keys at each level: both keys in one call, and each key in
    its own call as the benchmark times them."""
    c = cases.case_n16_level(level)
    want = digests[c.name]["digests"]
    prm = params_for(c, max_batch=8, max_hoist=2)
    check_items(c, run_case(prm, c), want, f"level {level}, both keys", oracle_item=oracle_of(c))
    ct = dev(c.cts)
    for r, k in enumerate(c.keys):
        out = host(ksa.keyswitch_ex(prm, ct, [dev(k.b)], [k.galois], level, seeds=[k.seed]))[0]
        check_items(c, None, want, f"level {level}, key {r} alone",
                    index=[(r * c.batch + b, out[b]) for b in range(c.batch)])
    prm.close()


def test_n16_extreme_inputs_every_item(digests):
    """All-0, all-(q-1) and largest-ModUp-coefficient ciphertexts beside uniform ones,
    under a key whose b words are all r-1 (a regenerated) and a conjugation key whose
    stored b and a have the largest Montgomery-form value, at k = 8 and k = 1."""
    cx, cy = cases.case_n16_extreme()
    prm = params_for(cx, max_batch=8)
    for c in (cx, cy):
        want = digests[c.name]["digests"]
        check_items(c, run_case(prm, c), want, f"{c.name} k=8", oracle_item=oracle_of(c))
        check_items(c, run_case(prm, c, single=True), want, f"{c.name} k=1", oracle_item=oracle_of(c))
    prm.close()


def test_n17_relinearise_then_rotate_every_item(digests):
    """N=2^17, L=40, dnum=5, K=8: all 8 ciphertexts after the relinearisation and
    after the X^5 rotation of the result; then the rotation of one ciphertext alone
    (the segment-layout gathers)."""
    c = cases.case_n17_chain()
    want = digests[c.name]["digests"]
    relin, rot = c.keys
    prm = params_for(c, max_batch=8)
    step1 = ksa.keyswitch_ex(prm, dev(c.cts), [dev(relin.b)], [1], c.level, seeds=[relin.seed])
    s1 = host(step1)[0]
    step2 = host(ksa.keyswitch_ex(prm, step1[0].contiguous(), [dev(rot.b)], [5], c.level, seeds=[rot.seed]))[0]

    def oracle_item(idx):
        b = idx % 8
        first = ks.keyswitch(c.prm, c.cts[b], relin, c.level)
        return first if idx < 8 else ks.keyswitch(c.prm, first, rot, c.level)

    check_items(c, None, want, "relinearisation", index=[(b, s1[b]) for b in range(8)], oracle_item=oracle_item)
    check_items(c, None, want, "rotation", index=[(8 + b, step2[b]) for b in range(8)], oracle_item=oracle_item)
    one = host(ksa.keyswitch(prm, step1[0][5].contiguous(), dev(rot.b), rot.seed, c.level, 5))
    check_items(c, None, want, "single rotation", index=[(13, one)], oracle_item=oracle_item)
    prm.close()


def test_n17_rotation_batch7_matches_single_calls():
    """A batch of 7 under the X^5 key at N=2^17 gathers from more than 16 MB of
    sources per limb and takes the inner product's one-workgroup-per-unit kernel
    with each thread expanding its ChaCha blocks, at a batch size the kernel is
    not specialised for. Every item must equal the single-ciphertext call on it,
    the path that the chain's digests pin to the oracle (item 13 above)."""
    c = cases.case_n17_chain()
    rot = c.keys[1]
    prm = params_for(c, max_batch=8)
    kb = dev(rot.b)
    cts = dev(c.cts[:7])
    batch = host(ksa.keyswitch_ex(prm, cts, [kb], [5], c.level, seeds=[rot.seed]))[0]
    for b in range(7):
        one = host(ksa.keyswitch(prm, cts[b].contiguous(), kb, rot.seed, c.level, 5))
        diff = np.flatnonzero(batch[b].reshape(-1) != one.reshape(-1))
        assert diff.size == 0, f"item {b}: {diff.size} words differ from the single call, first at {diff[0]}"
    prm.close()


def test_n16_live_oracle_item_and_decryption():
    """One item compared word for word with a live oracle run, and its decryption under
    the real secret within the bound (the digests pin the rest)."""
    c = cases.case_n16_relin_k8()
    s, key, emax = cases.n16_relin_key(c.prm)
    prm = params_for(c, max_batch=8)
    out = host(ksa.keyswitch_ex(prm, dev(c.cts), [dev(key.b)], [1], c.level, seeds=[key.seed]))[0]
    ref = ks.keyswitch(c.prm, c.cts[6], key, c.level)
    diff = np.flatnonzero(out[6].astype(np.uint64).reshape(-1) != ref.reshape(-1))
    assert diff.size == 0, f"item 6: {diff.size} words differ, first at {diff[0]}"
    e = ks.decryption_error(c.prm, c.cts[6], out[6], s, 1, c.level)
    w = ki.WORKLOADS["n16"]
    assert e is not None and np.abs(e).max() <= ks.error_bound(c.prm, c.level, emax, w.h)
    prm.close()
