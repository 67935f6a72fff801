"""ChaCha block function and the key-half expander (oracle; test infrastructure only).

Per the Perseus README ('What's inside'), the GPU re-creates one of the two
halves of each key-switching key from a ChaCha12 seed, so that half never
sits in memory; the arXiv summary page (methodology, item (i)) describes the
generator as ChaCha12 run in counter mode. The pages fix neither the state layout nor how keystream words
become residues. Reading taken here:

* state: the standard ChaCha layout -- four constant words spelling
  "expand 32-byte k", the 256-bit seed as eight little-endian words, a 32-bit
  block counter starting at 0 (word 12) and three nonce words (13, 14, 15) =
  (0, d, j), with d the digit and j the limb's index in the key basis;
* ChaCha12 = 6 double rounds (a column round then a diagonal round), output =
  final working state + input state (word-wise mod 2^32);
* value i of limb j of digit d = (w[2i] + 2^32 w[2i+1]) mod r_j, where w[16b+o]
  is word o of block b; so block b covers values 8b..8b+7, and 'a' is drawn
  directly in the evaluation domain (value i is evaluation position i).

Rounds are a parameter so that the same code at 20 rounds can be compared
with the ChaCha20 of the OpenSSL command line.
"""

from __future__ import annotations

import numpy as np

SIGMA_WORDS = (0x61707865, 0x3320646E, 0x79622D32, 0x6B206574)  # "expand 32-byte k"


def _rotl(x: np.ndarray, n: int) -> np.ndarray:
    return (x << np.uint32(n)) | (x >> np.uint32(32 - n))


def _quarter_round(x: list, a: int, b: int, c: int, d: int) -> None:
    x[a] = x[a] + x[b]
    x[d] = _rotl(x[d] ^ x[a], 16)
    x[c] = x[c] + x[d]
    x[b] = _rotl(x[b] ^ x[c], 12)
    x[a] = x[a] + x[b]
    x[d] = _rotl(x[d] ^ x[a], 8)
    x[c] = x[c] + x[d]
    x[b] = _rotl(x[b] ^ x[c], 7)


def chacha_blocks(key: bytes, nonce: tuple, counters: np.ndarray, rounds: int = 12) -> np.ndarray:
    """Keystream blocks [len(counters)][16] uint32 for a 32-byte key and 3-word nonce."""
    if len(key) != 32:
        raise ValueError("key must be 32 bytes")
    if rounds % 2:
        raise ValueError("rounds must be even (whole double rounds)")
    counters = np.asarray(counters, dtype=np.uint32)
    nb = counters.shape[0]
    kw = np.frombuffer(key, dtype="<u4")
    init = [np.full(nb, w, dtype=np.uint32) for w in SIGMA_WORDS]
    init += [np.full(nb, kw[i], dtype=np.uint32) for i in range(8)]
    init += [counters.copy()]
    init += [np.full(nb, int(n) & 0xFFFFFFFF, dtype=np.uint32) for n in nonce]
    x = [w.copy() for w in init]
    with np.errstate(over="ignore"):
        for _ in range(rounds // 2):
            _quarter_round(x, 0, 4, 8, 12)
            _quarter_round(x, 1, 5, 9, 13)
            _quarter_round(x, 2, 6, 10, 14)
            _quarter_round(x, 3, 7, 11, 15)
            _quarter_round(x, 0, 5, 10, 15)
            _quarter_round(x, 1, 6, 11, 12)
            _quarter_round(x, 2, 7, 8, 13)
            _quarter_round(x, 3, 4, 9, 14)
        out = np.stack([x[i] + init[i] for i in range(16)], axis=1)
    return out


def keystream_words(key: bytes, nonce: tuple, nwords: int, rounds: int = 12) -> np.ndarray:
    """The first ``nwords`` stream words w[0..nwords) (counter from 0)."""
    nb = (nwords + 15) // 16
    return chacha_blocks(key, nonce, np.arange(nb, dtype=np.uint32), rounds).reshape(-1)[:nwords]


def expand_uniform(seed: bytes, d: int, j: int, N: int, r: int, rounds: int = 12) -> np.ndarray:
    """Limb j of digit d of a key's regenerated half: N residues mod r (uint64)."""
    w = keystream_words(seed, (0, d, j), 2 * N, rounds).astype(np.uint64)
    lo = w[0::2]
    hi = w[1::2]
    return ((hi << np.uint64(32)) | lo) % np.uint64(r)
