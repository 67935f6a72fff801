"""The fused ModUp/inner-product tile at N = 2^16 for every digit count.

One key of Galois element 1 (the relinearisation shape) takes the fused tile
(ModUp's block pass and the inner product in one kernel); at N = 2^16 its tile
is 16 columns wide with the twiddles on chip. The full-size workloads reach it
only with four digits (level 24), so this test runs one relinearisation key at
levels whose digit counts are 1 to 4, with full and ragged last digits, at
batch 3 and batch 1, with the a half regenerated and stored, and compares
every output item word for word with a live run of the oracle (the uniform key
halves of the full-size recipe; inputs from ks_inputs). At N = 2^17 the tile
has 8 columns and loads its twiddles per round; it is checked at three levels
below the top one against the C++ oracle tier.
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

# level -> digits at N = 2^16, L = 24, dnum = 4 (ceil(l/4) primes per digit at
# level l): 5+5+5+4, 4+4+4+1, 3+3+3, 2+2+1, 1+1, 1
LEVELS = {19: 4, 13: 4, 9: 3, 5: 3, 2: 2, 1: 1}


@pytest.fixture(scope="module")
def prm():
    assert torch.cuda.is_available(), "these tests need the GPU"
    torch.cuda.set_device(0)
    oprm = cases.n16_params()
    p = ksa.Params(oprm.log2n, oprm.L, oprm.dnum, oprm.K, device=0, max_batch=3)
    assert tuple(p.primes) == oprm.primes
    yield oprm, p
    torch.cuda.synchronize()
    p.close()


@pytest.mark.parametrize("level", sorted(LEVELS))
def test_fused_tile_every_digit_count(prm, level):
    oprm, p = prm
    assert len(oprm.digits(level)) == LEVELS[level]
    widx = ki.WORKLOADS["n16"].index * 1000 + level
    cts = ki.ciphertexts(widx, oprm.q[:level], oprm.N, 3)
    key = cases.uniform_keys(oprm, widx, level, [1])[0]
    want = [ks.keyswitch(oprm, cts[b], key, level) for b in range(3)]
    kb = [ksa.to_device(key.b, 0)]
    ka = [ksa.to_device(ks.key_a(oprm, key), 0)]
    runs = {
        "regenerated a, batch 3": ksa.keyswitch_ex(p, ksa.to_device(cts, 0), kb, [1], level, seeds=[key.seed]),
        "stored a, batch 3": ksa.keyswitch_ex(p, ksa.to_device(cts, 0), kb, [1], level, evk_a=ka),
        "regenerated a, batch 1": ksa.keyswitch_ex(p, ksa.to_device(cts[1:2], 0), kb, [1], level, seeds=[key.seed]),
    }
    torch.cuda.synchronize()
    for label, out in runs.items():
        got = ksa.to_host(out)[0]
        items = [1] if got.shape[0] == 1 else range(3)
        for i, b in enumerate(items):
            diff = np.flatnonzero(got[i].astype(np.uint64).reshape(-1) != want[b].reshape(-1))
            assert diff.size == 0, (f"level {level} ({LEVELS[level]} digits), {label}, item {b}: "
                                    f"{diff.size} words differ from the oracle, first at {diff[0]}")


@pytest.mark.parametrize("level", [24, 9])
def test_fused_tile_chacha20(level):
    """The same tile with the a half expanded by ChaCha20 (the 20-round build of
    the expander), against the oracle with the same round count."""
    assert torch.cuda.is_available(), "these tests need the GPU"
    torch.cuda.set_device(0)
    oprm = ks.Params(16, 24, 4, 6, chacha_rounds=20)
    p = ksa.Params(16, 24, 4, 6, device=0, chacha_rounds=20, max_batch=3)
    try:
        assert tuple(p.primes) == oprm.primes
        widx = ki.WORKLOADS["n16"].index * 1000 + 500 + level
        cts = ki.ciphertexts(widx, oprm.q[:level], oprm.N, 3)
        key = cases.uniform_keys(oprm, widx, level, [1])[0]
        out = ksa.keyswitch_ex(p, ksa.to_device(cts, 0), [ksa.to_device(key.b, 0)], [1], level, seeds=[key.seed])
        torch.cuda.synchronize()
        got = ksa.to_host(out)[0]
        for b in range(3):
            want = ks.keyswitch(oprm, cts[b], key, level)
            diff = np.flatnonzero(got[b].astype(np.uint64).reshape(-1) != want.reshape(-1))
            assert diff.size == 0, f"level {level}, ChaCha20, item {b}: {diff.size} words differ, first at {diff[0]}"
    finally:
        torch.cuda.synchronize()
        p.close()


# N = 2^17, L = 40, dnum = 5, K = 8 (the 8-column tile with per-round twiddle
# loads): 7+7+7+7+5, 2+2+2+2 and 1+1+1 primes per digit
N17_LEVELS = {33: 5, 8: 4, 3: 3}


@pytest.mark.parametrize("level", sorted(N17_LEVELS))
def test_fused_tile_n17_levels(level):
    """One relinearisation key at N = 2^17 below the top level, batch 2, against the
    C++ oracle tier (equal to the numpy oracle word for word, pinned by the CPU
    tests; used here for its speed at this ring size)."""
    from oracle import o2
    assert torch.cuda.is_available(), "these tests need the GPU"
    torch.cuda.set_device(0)
    oprm = cases.n17_params()
    assert len(oprm.digits(level)) == N17_LEVELS[level]
    O = o2.O2(oprm.log2n, oprm.L, oprm.dnum, oprm.K)
    p = ksa.Params(oprm.log2n, oprm.L, oprm.dnum, oprm.K, device=0, max_batch=2)
    try:
        assert tuple(p.primes) == oprm.primes and tuple(O.primes) == oprm.primes
        widx = ki.WORKLOADS["n17"].index * 1000 + level
        cts = ki.ciphertexts(widx, oprm.q[:level], oprm.N, 2)
        key = cases.uniform_keys(oprm, widx, level, [1])[0]
        out = ksa.keyswitch_ex(p, ksa.to_device(cts, 0), [ksa.to_device(key.b, 0)], [1], level, seeds=[key.seed])
        torch.cuda.synchronize()
        got = ksa.to_host(out)[0]
        for b in range(2):
            want = O.keyswitch(cts[b], level, 1, key.b, seed=key.seed)
            diff = np.flatnonzero(got[b].reshape(-1) != want.reshape(-1))
            assert diff.size == 0, f"N=2^17 level {level}, item {b}: {diff.size} words differ, first at {diff[0]}"
    finally:
        torch.cuda.synchronize()
        p.close()
        O.close()
