"""Loader of the C++ oracle tier, ks_o2.cpp (oracle; test infrastructure only).

ks_o2.cpp computes the same key switch as ``oracle.keyswitch`` from the same
definitions, in plain C++17 with OpenMP over independent (digit, limb) items,
sharing no code with it or with the GPU library. Two oracles written apart
check each other: the tests compare them word for word on small random shapes
and at the full sizes, and the benchmark times this one as the CPU baseline.
This module only builds the shared object with g++ and marshals arrays through
ctypes; every step of the arithmetic is in ks_o2.cpp.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ks_o2.cpp")
LIB = os.path.join(HERE, "libks_o2.so")
FLAGS = ["-O2", "-std=c++17", "-fopenmp", "-shared", "-fPIC"]

_lib = None


def build(verbose: bool = False) -> str:
    """Compile ks_o2.cpp into oracle/libks_o2.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = ["g++", *FLAGS, SRC, "-o", tmp]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"g++ failed ({res.returncode}):\n{res.stdout}")
    os.replace(tmp, LIB)
    if verbose:
        print(" ".join(cmd), flush=True)
    return LIB


def lib() -> ctypes.CDLL:
    """The loaded library; built first if it is missing or older than its source."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB)
        vp, u32p, u8p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint32), ctypes.c_char_p
        L.o2_create.restype = vp
        L.o2_create.argtypes = [ctypes.c_int] * 6
        L.o2_destroy.argtypes = [vp]
        L.o2_tables.argtypes = [vp, u32p, u32p]
        L.o2_ntt.restype = ctypes.c_int
        L.o2_ntt.argtypes = [vp, ctypes.c_int, u32p, ctypes.c_int]
        L.o2_chacha_blocks.argtypes = [u8p, ctypes.c_uint32, u32p, ctypes.c_int, ctypes.c_int, u32p]
        L.o2_keyswitch.restype = ctypes.c_int
        L.o2_keyswitch.argtypes = [vp, ctypes.c_int, u32p, ctypes.c_uint32, u32p, u32p, u8p, u32p, ctypes.c_int]
        _lib = L
    return _lib


def _u32(a) -> np.ndarray:
    a = np.asarray(a)
    if a.size and int(a.max()) >= (1 << 32):
        raise ValueError("words must fit in 32 bits")
    return np.ascontiguousarray(a, dtype=np.uint32)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32))


class O2:
    """A parameter set of the C++ oracle (same meaning as ``oracle.keyswitch.Params``)."""

    def __init__(self, log2n: int, L: int, dnum: int, K: int, partition: int = 0, rounds: int = 12):
        self.log2n, self.L, self.dnum, self.K, self.partition = log2n, L, dnum, K, partition
        self.N = 1 << log2n
        self._h = lib().o2_create(log2n, L, dnum, K, partition, rounds)
        if not self._h:
            raise ValueError(f"o2_create rejected log2n={log2n} L={L} dnum={dnum} K={K} "
                             f"partition={partition} rounds={rounds}")
        self.primes, self.psi = self.tables()

    def close(self):
        if self._h:
            lib().o2_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def tables(self):
        """(primes, psi) as lists: L q-primes then K p-primes, and each one's root."""
        n = self.L + self.K
        pr, ps = np.zeros(n, dtype=np.uint32), np.zeros(n, dtype=np.uint32)
        lib().o2_tables(self._h, _ptr(pr), _ptr(ps))
        return [int(x) for x in pr], [int(x) for x in ps]

    def ntt(self, x, k: int, inverse: bool = False) -> np.ndarray:
        """Forward (or inverse) negacyclic NTT of one limb mod prime k."""
        a = _u32(x).copy()
        if a.shape != (self.N,):
            raise ValueError("one limb of N words expected")
        if lib().o2_ntt(self._h, k, _ptr(a), int(inverse)) != 0:
            raise ValueError(f"prime index {k} out of range")
        return a

    def keyswitch(self, ct, level: int, galois: int, evk_b, seed: bytes = None, evk_a=None,
                  threads: int = 0, validate: bool = True) -> np.ndarray:
        """ct [2][level][N] -> [2][level][N]; evk_b (and evk_a) [beta_key][key_level+K][N].

        validate=False skips the scan for non-canonical words (for timing loops over
        inputs already checked once); shapes are always checked."""
        if validate:
            ct, b = _u32(ct), _u32(evk_b)
            a = _u32(evk_a) if evk_a is not None else None
        else:
            ct, b = np.ascontiguousarray(ct, dtype=np.uint32), np.ascontiguousarray(evk_b, dtype=np.uint32)
            a = np.ascontiguousarray(evk_a, dtype=np.uint32) if evk_a is not None else None
        if ct.shape != (2, level, self.N):
            raise ValueError(f"ciphertext shape {ct.shape} != (2, {level}, {self.N})")
        kl = self.L if self.partition else level
        if b.ndim != 3 or b.shape[1:] != (kl + self.K, self.N):
            raise ValueError(f"key shape {b.shape} does not match key level {kl}")
        if a is not None and a.shape != b.shape:
            raise ValueError("stored a half must have the b half's shape")
        if a is None and (seed is None or len(seed) != 32):
            raise ValueError("a 32-byte seed or a stored a half is needed")
        primes = self.primes
        q = np.array(primes[:level], dtype=np.uint32)[:, None]
        key_basis = np.array(primes[:kl] + primes[self.L:], dtype=np.uint32)[:, None]
        if validate and ((ct >= q).any() or (b >= key_basis).any() or (a is not None and (a >= key_basis).any())):
            raise ValueError("words must be canonical residues (below their limb's prime)")
        alpha = -(-(self.L if self.partition else level) // self.dnum)
        if b.shape[0] < -(-level // alpha):
            raise ValueError("the key has fewer digits than the level needs")
        out = np.empty((2, level, self.N), dtype=np.uint32)
        rc = lib().o2_keyswitch(self._h, level, _ptr(ct), galois, _ptr(b), _ptr(a) if a is not None else None,
                                seed if a is None else None, _ptr(out), threads)
        if rc != 0:
            raise ValueError(f"o2_keyswitch rejected level={level} galois={galois}")
        return out


def chacha_blocks(key: bytes, counter: int, nonce, nblocks: int, rounds: int = 12) -> np.ndarray:
    """[nblocks][16] keystream words from the C++ oracle's block function."""
    if len(key) != 32:
        raise ValueError("key must be 32 bytes")
    nw = np.asarray(nonce, dtype=np.uint32)
    out = np.empty((nblocks, 16), dtype=np.uint32)
    lib().o2_chacha_blocks(key, counter, _ptr(nw), rounds, nblocks, _ptr(out))
    return out
