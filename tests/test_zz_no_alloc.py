"""pc_keyswitch_static (the entry point that allocates nothing) against pc_keyswitch_ex.

Two calls in a row through the C ABI, the second with a smaller input (a lower
level, so less of the shared scratch is written and the first call's contents
stay in the rest of it), then a third with one relinearisation key (the fused
ModUp/inner-product tile); every output word must equal pc_keyswitch_ex's on
the same inputs. Shapes whose workspace exceeds the scratch are refused.
"""

import numpy as np
import pytest

import ks_inputs as ki

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ksa = pytest.importorskip("key_switching_amd")


def _host(t):
    torch.cuda.synchronize()
    return ksa.to_host(t)


def test_static_matches_ex_on_two_calls_the_second_smaller():
    assert torch.cuda.is_available()
    torch.cuda.set_device(0)
    w = ki.WORKLOADS["n16"]
    prm = ksa.Params(w.log2n, w.L, w.dnum, w.K, max_batch=8, max_hoist=2, device=0)
    q = prm.primes[: w.L]
    # two keys at level 24, then one key at level 12, then the relinearisation key at level 20
    calls = [(w.L, [1, 5]), (12, [2 * w.N - 1]), (20, [1])]
    for n, (level, galois) in enumerate(calls):
        basis, beta = prm.basis(level), prm.beta(level)
        keys = [ksa.to_device(ki.uniform_key_b(90 + n, k, beta, basis, w.N), 0) for k in range(len(galois))]
        seeds = [ki.key_seed(90 + n, k) for k in range(len(galois))]
        ct = ksa.to_device(ki.ciphertexts(90 + n, q[:level], w.N, 1), 0)
        out = torch.empty((len(galois), 1, 2, level, w.N), dtype=torch.int32, device="cuda:0")
        ksa.keyswitch_static(prm, ct, keys, galois, level, seeds=seeds, out=out)
        got = _host(out)
        want = _host(ksa.keyswitch_ex(prm, ct, keys, galois, level, seeds=seeds))
        bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
        assert bad.size == 0, f"call {n} (level {level}): {bad.size} words differ, first at {bad[:1]}"
    # a batch of 8 at the top level needs more than the scratch holds
    ct8 = ksa.to_device(ki.ciphertexts(99, q, w.N, 8), 0)
    key = ksa.to_device(ki.uniform_key_b(99, 0, prm.beta(w.L), prm.basis(w.L), w.N), 0)
    with pytest.raises(ksa.PcError) as e:
        ksa.keyswitch_static(prm, ct8, [key], [1], w.L, seeds=[ki.key_seed(99, 0)])
    assert e.value.code == ksa.PC_EUNSUPPORTED
    prm.close()
