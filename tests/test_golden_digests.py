"""The stored full-size digests are the oracle's (CPU).

tests/golden/digests_full.json holds one SHA-256 per output item of the
full-size cases; the GPU tests compare against it. Here: the file was written
from the current oracle, input generators and recipe (their hash), it covers
every case and item, and a sample of its entries recomputed by the oracle now
agrees with it.
"""

import os
import sys

import pytest

from oracle import keyswitch as ks

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden"))
import cases  # noqa: E402


@pytest.fixture(scope="module")
def doc():
    return cases.load_digests()


def test_digests_written_from_current_sources(doc):
    assert doc["sources_hash"] == cases.sources_hash(), "run tests/golden/make_digests.py"


def test_every_case_and_item_present(doc):
    want = {"n16_relin_k8": 8, "n16_hoist16": 16, "n16_extreme_x": 8, "n16_extreme_y": 8, "n17_chain": 16}
    want.update({f"n16_level{lv}": 16 for lv in cases.LEVELS})
    assert set(doc["cases"]) == set(want)
    for name, n in want.items():
        d = doc["cases"][name]["digests"]
        assert len(d) == n and len(set(d)) == n, name  # distinct inputs give distinct outputs


@pytest.mark.parametrize("item", [0, 5])
def test_level4_entries_recomputed(doc, item):
    """Level 4 is the cheapest full-size case: both keys of two ciphertexts, run again."""
    c = cases.case_n16_level(4)
    outs = ks.keyswitch_hoisted(c.prm, c.cts[item], c.keys, c.level)
    want = doc["cases"]["n16_level4"]["digests"]
    for r, o in enumerate(outs):
        assert cases.digest(o) == want[r * c.batch + item]


def test_extreme_inputs_are_extreme():
    """The recipe's special ciphertexts and keys hold the words they claim to hold."""
    cx, cy = cases.case_n16_extreme()
    q = cx.prm.q
    assert (cx.cts[0] == 0).all()
    for i in range(cx.level):
        assert (cx.cts[1, :, i] == q[i] - 1).all()
    basis = cx.prm.basis(cx.level)
    for j, r in enumerate(basis):
        assert (cx.keys[0].b[:, j] == r - 1).all()
        m = cy.keys[0].b[0, j, 0]
        assert (int(m) * pow(2, -32, r)) % r == r - 1
        assert (cy.keys[0].a[:, j] == m).all()
    # ciphertext 2: ModUp's scaled coefficients are q_i - 1 at every position
    from oracle import rns
    import math
    prm = cx.prm
    for D in prm.digits(cx.level):
        Qd = math.prod(prm.q[i] for i in D)
        i = D[-1]
        y = rns.intt(cx.cts[2, 1, i], q[i]) * pow((Qd // q[i]) % q[i], -1, q[i]) % q[i]
        assert (y == q[i] - 1).all()
