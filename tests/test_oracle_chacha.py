"""Pins of the oracle's ChaCha block function and key-half expander (CPU only).

At 20 rounds the oracle's keystream is compared with the ChaCha20 of the
OpenSSL command line (its 16-byte IV is the little-endian 32-bit block
counter followed by the 96-bit nonce). At 0 rounds the output is twice the
input state, which pins the state layout (constants, key words, counter,
nonce) independently of the round function. ChaCha12 itself has no external
vector here: it is the same double round, iterated 6 times instead of 10.
"""

import random
import shutil
import subprocess

import numpy as np
import pytest

from oracle import chacha

HAVE_OPENSSL = shutil.which("openssl") is not None


def openssl_chacha20(key: bytes, counter: int, nonce_words, nbytes: int) -> bytes:
    iv = counter.to_bytes(4, "little") + b"".join(int(w).to_bytes(4, "little") for w in nonce_words)
    res = subprocess.run(
        ["openssl", "enc", "-chacha20", "-K", key.hex(), "-iv", iv.hex()],
        input=bytes(nbytes), stdout=subprocess.PIPE, stderr=subprocess.PIPE, check=True)
    assert len(res.stdout) == nbytes
    return res.stdout


@pytest.mark.skipif(not HAVE_OPENSSL, reason="openssl command line not available")
@pytest.mark.parametrize("case", range(6))
def test_chacha20_matches_openssl(case):
    rnd = random.Random(case)
    key = bytes(rnd.randrange(256) for _ in range(32)) if case else bytes(32)
    nonce = (0, rnd.randrange(8), rnd.randrange(64)) if case % 2 else tuple(rnd.randrange(1 << 32) for _ in range(3))
    counter = 0 if case < 3 else rnd.randrange(1 << 20)
    nblocks = 5
    ours = chacha.chacha_blocks(key, nonce, np.arange(counter, counter + nblocks, dtype=np.uint32), rounds=20)
    ref = np.frombuffer(openssl_chacha20(key, counter, nonce, 64 * nblocks), dtype="<u4").reshape(nblocks, 16)
    assert np.array_equal(ours, ref)


@pytest.mark.skipif(not HAVE_OPENSSL, reason="openssl command line not available")
def test_expander_word_pairs_against_openssl_bytes():
    """Value i = 64-bit little-endian word at stream bytes [8i, 8i+8) mod r (20 rounds)."""
    seed = bytes(range(32))
    N, r, d, j = 64, 2147377153, 2, 5
    vals = chacha.expand_uniform(seed, d, j, N, r, rounds=20)
    stream = openssl_chacha20(seed, 0, (0, d, j), 8 * N)
    ref = [int.from_bytes(stream[8 * i: 8 * i + 8], "little") % r for i in range(N)]
    assert vals.tolist() == ref


def test_zero_rounds_is_twice_the_state():
    key = bytes(range(100, 132))
    out = chacha.chacha_blocks(key, (7, 8, 9), np.array([3, 4], dtype=np.uint32), rounds=0)
    kw = [int.from_bytes(key[4 * i: 4 * i + 4], "little") for i in range(8)]
    for b, ctr in enumerate((3, 4)):
        state = [0x61707865, 0x3320646E, 0x79622D32, 0x6B206574] + kw + [ctr, 7, 8, 9]
        assert out[b].tolist() == [(2 * s) & 0xFFFFFFFF for s in state]


def test_rounds_change_the_stream():
    key = bytes(32)
    s12 = chacha.keystream_words(key, (0, 0, 0), 64, rounds=12)
    s20 = chacha.keystream_words(key, (0, 0, 0), 64, rounds=20)
    s8 = chacha.keystream_words(key, (0, 0, 0), 64, rounds=8)
    assert not np.array_equal(s12, s20) and not np.array_equal(s12, s8)


def test_expander_is_counter_mode():
    """Block b of limb (d, j) depends only on (seed, d, j, b): a prefix is a prefix."""
    seed = bytes(range(32))
    r = 2147352577
    long = chacha.expand_uniform(seed, 1, 3, 256, r)
    short = chacha.expand_uniform(seed, 1, 3, 64, r)
    assert np.array_equal(long[:64], short)
    other = chacha.expand_uniform(seed, 1, 4, 64, r)
    assert not np.array_equal(other, short)
    assert int(long.max()) < r


def test_expander_is_uniform_enough():
    r = 2102788097
    v = chacha.expand_uniform(bytes(32), 0, 0, 1 << 14, r).astype(np.float64) / r
    assert abs(v.mean() - 0.5) < 0.01
    hist, _ = np.histogram(v, bins=16, range=(0, 1))
    assert hist.min() > 0.8 * (1 << 14) / 16
