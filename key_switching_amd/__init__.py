"""Python binding of libpc.so, the gfx950 CKKS hybrid key-switching library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/pc.h. Device buffers are
PyTorch tensors (torch.int32 storage holding uint32 residues) and calls are
enqueued on the current PyTorch stream. The module raises if the shared
library has not been built (``python -m key_switching_amd.build``); there is
no CPU fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpc.so")

PC_OK, PC_EINVAL, PC_ENOMEM, PC_EDEVICE, PC_EUNSUPPORTED = 0, -1, -2, -3, -4
(PC_GET_N, PC_GET_PRIMES, PC_GET_PSI, PC_GET_ALPHA, PC_GET_BETA, PC_GET_WORKSPACE_BYTES, PC_GET_DEVICE_TABLE,
 PC_GET_ARENA_BYTES, PC_GET_LT_WORKSPACE_BYTES) = range(1, 10)

PC_KEYSET_PACKED, PC_KEYSET_FULL = 0, 1
PC_KEYSET_DEVICE_BYTES, PC_KEYSET_KEY_BYTES, PC_KEYSET_GALOIS, PC_KEYSET_B_POINTER = 1, 2, 3, 4

EXPORTED = ("pc_params_create", "pc_params_destroy", "pc_params_get", "pc_ntt", "pc_intt", "pc_modup",
            "pc_keyswitch", "pc_moddown", "pc_keyswitch_ex", "pc_keygen", "pc_tensor", "pc_rescale",
            "pc_hmult", "pc_linear_transform", "pc_chacha_expand",
            "pc_keyset_create", "pc_keyset_destroy", "pc_keyset_set", "pc_keyset_keygen", "pc_keyset_get",
            "pc_keyswitch_keyset", "pc_keyswitch_static",
            "pc_profile_begin", "pc_profile_end", "pc_strerror")


class PcError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {_lib().pc_strerror(code).decode()} ({code})")
        self.code = code


class _Desc(ctypes.Structure):
    _fields_ = [("log2n", ctypes.c_uint32), ("L", ctypes.c_uint32), ("dnum", ctypes.c_uint32),
                ("K", ctypes.c_uint32), ("max_batch", ctypes.c_uint32), ("max_hoist", ctypes.c_uint32),
                ("chacha_rounds", ctypes.c_uint32), ("partition", ctypes.c_uint32),
                ("primes", ctypes.POINTER(ctypes.c_uint32))]


class _KsArgs(ctypes.Structure):
    _fields_ = [("ct", ctypes.c_void_p), ("batch", ctypes.c_uint32), ("nkeys", ctypes.c_uint32),
                ("evk_b", ctypes.POINTER(ctypes.c_void_p)), ("evk_a", ctypes.POINTER(ctypes.c_void_p)),
                ("seeds", ctypes.c_char_p), ("galois", ctypes.POINTER(ctypes.c_uint32)),
                ("level", ctypes.c_uint32), ("out", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


class _LtArgs(ctypes.Structure):
    _fields_ = [("ct", ctypes.c_void_p), ("level", ctypes.c_uint32), ("n1", ctypes.c_uint32),
                ("n2", ctypes.c_uint32), ("diag", ctypes.c_void_p),
                ("baby_b", ctypes.POINTER(ctypes.c_void_p)), ("baby_seeds", ctypes.c_char_p),
                ("baby_galois", ctypes.POINTER(ctypes.c_uint32)),
                ("giant_b", ctypes.POINTER(ctypes.c_void_p)), ("giant_seeds", ctypes.c_char_p),
                ("giant_galois", ctypes.POINTER(ctypes.c_uint32)), ("out", ctypes.c_void_p)]


class _KStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_uint32), ("total_ms", ctypes.c_double)]


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m key_switching_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, u32, i32 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int
        lib.pc_params_create.argtypes = [ctypes.POINTER(_Desc), i32, ctypes.POINTER(vp)]
        lib.pc_params_destroy.argtypes = [vp]
        lib.pc_params_destroy.restype = None
        lib.pc_params_get.argtypes = [vp, i32, u32, vp, ctypes.c_size_t]
        lib.pc_ntt.argtypes = [vp, vp, ctypes.POINTER(u32), u32, u32, vp]
        lib.pc_intt.argtypes = [vp, vp, ctypes.POINTER(u32), u32, u32, vp]
        lib.pc_modup.argtypes = [vp, vp, u32, vp, vp]
        lib.pc_keyswitch.argtypes = [vp, vp, vp, ctypes.c_char_p, u32, u32, vp, vp]
        lib.pc_moddown.argtypes = [vp, vp, u32, vp, vp]
        lib.pc_keyswitch_ex.argtypes = [vp, ctypes.POINTER(_KsArgs), vp]
        lib.pc_keyswitch_static.argtypes = [vp, ctypes.POINTER(_KsArgs), vp]
        lib.pc_chacha_expand.argtypes = [vp, ctypes.c_char_p, u32, u32, u32, vp, vp]
        lib.pc_keygen.argtypes = [vp, ctypes.c_char_p, u32, u32, vp, vp, vp, vp]
        lib.pc_tensor.argtypes = [vp, vp, vp, u32, u32, vp, vp]
        lib.pc_rescale.argtypes = [vp, vp, u32, u32, vp, vp]
        lib.pc_hmult.argtypes = [vp, vp, vp, u32, vp, ctypes.c_char_p, u32, vp, vp]
        lib.pc_linear_transform.argtypes = [vp, ctypes.POINTER(_LtArgs), vp]
        lib.pc_keyset_create.argtypes = [vp, u32, u32, ctypes.POINTER(u32), u32, ctypes.POINTER(vp)]
        lib.pc_keyset_destroy.argtypes = [vp]
        lib.pc_keyset_destroy.restype = None
        lib.pc_keyset_set.argtypes = [vp, u32, vp, ctypes.c_char_p, vp]
        lib.pc_keyset_keygen.argtypes = [vp, u32, ctypes.c_char_p, vp, vp, vp]
        lib.pc_keyset_get.argtypes = [vp, i32, u32, vp, ctypes.c_size_t]
        lib.pc_keyswitch_keyset.argtypes = [vp, vp, vp, u32, ctypes.POINTER(u32), u32, u32, vp, vp,
                                            ctypes.c_size_t, vp]
        lib.pc_profile_begin.argtypes = [vp]
        lib.pc_profile_end.argtypes = [vp, ctypes.POINTER(_KStat), u32, ctypes.POINTER(u32)]
        lib.pc_strerror.argtypes = [i32]
        lib.pc_strerror.restype = ctypes.c_char_p
        for name in ("pc_params_create", "pc_params_get", "pc_ntt", "pc_intt", "pc_modup", "pc_keyswitch",
                     "pc_moddown", "pc_keyswitch_ex", "pc_chacha_expand", "pc_profile_begin", "pc_profile_end",
                     "pc_keygen", "pc_tensor", "pc_rescale", "pc_hmult", "pc_linear_transform",
                     "pc_keyset_create", "pc_keyset_set", "pc_keyset_keygen", "pc_keyset_get",
                     "pc_keyswitch_keyset", "pc_keyswitch_static"):
            getattr(lib, name).restype = i32
        _LIB = lib
    return _LIB


def _check(code: int, what: str):
    if code != PC_OK:
        raise PcError(code, what)


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev_ptr(t, name: str, shape=None, device=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA tensor")
    if t.dtype not in (torch.int32, torch.uint32):
        raise ValueError(f"{name} must hold 32-bit words (torch.int32 or torch.uint32)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if device is not None and t.device.index != device:
        raise ValueError(f"{name} is on cuda:{t.device.index}, the params on cuda:{device}")
    if t.data_ptr() % 16:
        raise ValueError(f"{name} must start at a 16-byte aligned address")
    return ctypes.c_void_p(t.data_ptr())


class Params:
    """Parameter set, constant tables and workspace arena (pc_params_create)."""

    def __init__(self, log2n: int, L: int, dnum: int, K: int, max_batch: int = 1, max_hoist: int = 1,
                 chacha_rounds: int = 12, primes: Optional[Sequence[int]] = None, device: Optional[int] = 0,
                 partition: int = 0):
        lib = _lib()
        desc = _Desc(log2n, L, dnum, K, max_batch, max_hoist, chacha_rounds, partition, None)
        self._primes_buf = None
        if primes is not None:
            self._primes_buf = (ctypes.c_uint32 * len(primes))(*[int(p) for p in primes])
            desc.primes = ctypes.cast(self._primes_buf, ctypes.POINTER(ctypes.c_uint32))
        self.device = -1 if device is None else int(device)
        h = ctypes.c_void_p()
        _check(lib.pc_params_create(ctypes.byref(desc), self.device, ctypes.byref(h)), "pc_params_create")
        self._h = h
        self.log2n, self.L, self.dnum, self.K = log2n, L, dnum, K
        self.max_batch, self.max_hoist = max_batch, max_hoist
        self.partition = partition

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("params closed")
        return self._h

    def close(self):
        if getattr(self, "_h", None) is not None:
            _lib().pc_params_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    @property
    def N(self) -> int:
        return 1 << self.log2n

    def _get_u32(self, what: int, arg: int = 0, count: int = 1):
        buf = (ctypes.c_uint32 * count)()
        _check(_lib().pc_params_get(self.handle, what, arg, buf, 4 * count), "pc_params_get")
        return list(buf)

    @property
    def primes(self):
        return self._get_u32(PC_GET_PRIMES, 0, self.L + self.K)

    @property
    def psi(self):
        return self._get_u32(PC_GET_PSI, 0, self.L + self.K)

    def alpha(self, level: int) -> int:
        return self._get_u32(PC_GET_ALPHA, level)[0]

    def key_level(self, level: int) -> int:
        """Level of the key that serves ciphertexts at ``level`` (L with partition 1)."""
        return self.L if self.partition else level

    def key_shape(self, level: int) -> tuple:
        """Shape of a key half serving ``level``: [beta(kl)][kl + K][N], kl = key_level(level)."""
        kl = self.key_level(level)
        return (self.beta(kl), kl + self.K, self.N)

    def beta(self, level: int) -> int:
        return self._get_u32(PC_GET_BETA, level)[0]

    def workspace_bytes(self, level: int) -> int:
        buf = ctypes.c_uint64()
        _check(_lib().pc_params_get(self.handle, PC_GET_WORKSPACE_BYTES, level, ctypes.byref(buf), 8),
               "pc_params_get")
        return int(buf.value)

    def _get_u64(self, what: int, arg: int) -> int:
        buf = ctypes.c_uint64()
        _check(_lib().pc_params_get(self.handle, what, arg, ctypes.byref(buf), 8), "pc_params_get")
        return int(buf.value)

    def arena_bytes(self) -> int:
        """Size of the workspace arena sized at creation."""
        return self._get_u64(PC_GET_ARENA_BYTES, 0)

    def lt_workspace_bytes(self, level: int, n1: int, n2: int) -> int:
        """Arena bytes a linear transform with n1 baby and n2 giant steps needs at ``level``."""
        if not (0 < level < 256 and 0 < n1 < 256 and 0 < n2 < 65536):
            raise ValueError("level, n1 or n2 out of range")
        return self._get_u64(PC_GET_LT_WORKSPACE_BYTES, level | (n1 << 8) | (n2 << 16))

    def twiddles(self, prime_index: int):
        return self._get_u32(PC_GET_DEVICE_TABLE, prime_index, self.N)

    def basis(self, level: int):
        """Moduli of the extended basis at this level: q_0..q_{level-1}, p_0..p_{K-1}."""
        pr = self.primes
        return pr[:level] + pr[self.L:]


def _new(shape, like_device: int):
    import torch
    return torch.empty(shape, dtype=torch.int32, device=f"cuda:{like_device}")


def _transform(prm: Params, data, prime_idx: Sequence[int], fn, name: str):
    n = len(prime_idx)
    idx = (ctypes.c_uint32 * n)(*[int(i) for i in prime_idx])
    if data.dim() == 2:
        count, shape = 1, (n, prm.N)
    else:
        count, shape = int(data.shape[0]), (int(data.shape[0]), n, prm.N)
    ptr = _dev_ptr(data, "data", shape, prm.device)
    _check(fn(prm.handle, ptr, idx, n, count, _stream()), name)
    return data


def ntt(prm: Params, data, prime_idx: Sequence[int]):
    """In-place negacyclic NTT (pc_ntt) of data [len(prime_idx)][N], or of
    [count][len(prime_idx)][N] (limb z of every polynomial uses prime_idx[z])."""
    return _transform(prm, data, prime_idx, _lib().pc_ntt, "pc_ntt")


def intt(prm: Params, data, prime_idx: Sequence[int]):
    """In-place inverse NTT (pc_intt); shapes as in ntt()."""
    return _transform(prm, data, prime_idx, _lib().pc_intt, "pc_intt")


def modup(prm: Params, c1, level: int, ext=None):
    """ModUp of c1 [level][N] into ext [beta][level+K][N] (pc_modup)."""
    shape = (prm.beta(level), level + prm.K, prm.N)
    if ext is None:
        ext = _new(shape, prm.device)
    _check(_lib().pc_modup(prm.handle, _dev_ptr(c1, "c1", (level, prm.N), prm.device), level,
                           _dev_ptr(ext, "ext", shape, prm.device), _stream()), "pc_modup")
    return ext


def moddown(prm: Params, acc, level: int, out=None):
    """ModDown of acc [level+K][N] into out [level][N] (pc_moddown)."""
    if out is None:
        out = _new((level, prm.N), prm.device)
    _check(_lib().pc_moddown(prm.handle, _dev_ptr(acc, "acc", (level + prm.K, prm.N), prm.device), level,
                             _dev_ptr(out, "out", (level, prm.N), prm.device), _stream()), "pc_moddown")
    return out


def _seed_bytes(seed) -> bytes:
    seed = bytes(seed)
    if len(seed) != 32:
        raise ValueError("a seed is 32 bytes")
    return seed


def keyswitch(prm: Params, ct, evk_b, seed: bytes, level: int, galois: int, out=None):
    """One key switch of ct [2][level][N] (pc_keyswitch)."""
    if out is None:
        out = _new((2, level, prm.N), prm.device)
    kshape = prm.key_shape(level)
    _check(_lib().pc_keyswitch(prm.handle, _dev_ptr(ct, "ct", (2, level, prm.N), prm.device),
                               _dev_ptr(evk_b, "evk_b", kshape, prm.device), _seed_bytes(seed), level, galois,
                               _dev_ptr(out, "out", (2, level, prm.N), prm.device), _stream()), "pc_keyswitch")
    return out


def _ks_call(fn, name, prm: Params, ct, evk_b: Sequence, galois: Sequence[int], level: int, seeds=None,
             evk_a=None, out=None, workspace=None):
    batch = int(ct.shape[0])
    nkeys = len(evk_b)
    if len(galois) != nkeys:
        raise ValueError("one Galois element per key")
    kshape = prm.key_shape(level)
    if out is None:
        out = _new((nkeys, batch, 2, level, prm.N), prm.device)
    args = _KsArgs()
    args.ct = _dev_ptr(ct, "ct", (batch, 2, level, prm.N), prm.device)
    args.batch = batch
    args.nkeys = nkeys
    b_ptrs = (ctypes.c_void_p * nkeys)(*[_dev_ptr(b, "evk_b", kshape, prm.device).value for b in evk_b])
    args.evk_b = b_ptrs
    a_ptrs = None
    if evk_a is not None:
        if len(evk_a) != nkeys:
            raise ValueError("one stored a half per key")
        a_ptrs = (ctypes.c_void_p * nkeys)(*[_dev_ptr(a, "evk_a", kshape, prm.device).value for a in evk_a])
        args.evk_a = a_ptrs
    seed_blob = None
    if seeds is not None:
        if len(seeds) != nkeys:
            raise ValueError("one seed per key")
        seed_blob = b"".join(_seed_bytes(s) for s in seeds)
        args.seeds = seed_blob
    gal = (ctypes.c_uint32 * nkeys)(*[int(g) for g in galois])
    args.galois = gal
    args.level = level
    args.out = _dev_ptr(out, "out", (nkeys, batch, 2, level, prm.N), prm.device)
    if workspace is not None:
        args.workspace = _dev_ptr(workspace, "workspace", None, prm.device)
        args.workspace_bytes = workspace.numel() * workspace.element_size()
    _check(fn(prm.handle, ctypes.byref(args), _stream()), name)
    return out


def keyswitch_ex(prm: Params, ct, evk_b: Sequence, galois: Sequence[int], level: int, seeds=None, evk_a=None,
                 out=None, workspace=None):
    """Every ciphertext of ct [batch][2][level][N] under every key (pc_keyswitch_ex).

    Returns out [nkeys][batch][2][level][N]. ``seeds`` lists one 32-byte seed
    per key (regenerated a half); ``evk_a`` lists stored a halves instead.
    """
    return _ks_call(_lib().pc_keyswitch_ex, "pc_keyswitch_ex", prm, ct, evk_b, galois, level, seeds, evk_a, out,
                    workspace)


def keyswitch_static(prm: Params, ct, evk_b: Sequence, galois: Sequence[int], level: int, seeds=None, evk_a=None,
                     out=None):
    """As keyswitch_ex, with the library's static scratch as the workspace
    (pc_keyswitch_static: no device allocation in the call; ``out`` must be
    given by callers that cannot allocate)."""
    return _ks_call(_lib().pc_keyswitch_static, "pc_keyswitch_static", prm, ct, evk_b, galois, level, seeds, evk_a,
                    out)


def keygen(prm: Params, seed: bytes, level: int, galois: int, s_coef, e_coef, out=None):
    """b half of a key at key level ``level`` for Galois element ``galois`` (pc_keygen).

    s_coef: [level+K][N] residues of the secret's coefficients mod each prime of
    the key basis; e_coef: [beta][level+K][N] residues of each digit's errors.
    Returns b [beta][level+K][N]; the a half is the ChaCha expansion of ``seed``.
    """
    lk = level + prm.K
    beta = prm.beta(level)
    if out is None:
        out = _new((beta, lk, prm.N), prm.device)
    _check(_lib().pc_keygen(prm.handle, _seed_bytes(seed), level, galois,
                            _dev_ptr(s_coef, "s_coef", (lk, prm.N), prm.device),
                            _dev_ptr(e_coef, "e_coef", (beta, lk, prm.N), prm.device),
                            _dev_ptr(out, "evk_b", (beta, lk, prm.N), prm.device), _stream()), "pc_keygen")
    return out


def _batched(t):
    """A [2][l][N] ciphertext as a batch of one (a view); [batch][2][l][N] unchanged."""
    return t.unsqueeze(0) if hasattr(t, "dim") and t.dim() == 3 else t


def tensor(prm: Params, ct_a, ct_b, level: int, out=None):
    """(d0, d1, d2) = (a0 b0, a0 b1 + a1 b0, a1 b1) per limb (pc_tensor).

    ct_a, ct_b: [batch][2][level][N] (or [2][level][N]); returns [batch][3][level][N].
    """
    ct_a, ct_b = _batched(ct_a), _batched(ct_b)
    batch = int(ct_a.shape[0])
    if out is None:
        out = _new((batch, 3, level, prm.N), prm.device)
    _check(_lib().pc_tensor(prm.handle, _dev_ptr(ct_a, "ct_a", (batch, 2, level, prm.N), prm.device),
                            _dev_ptr(ct_b, "ct_b", (batch, 2, level, prm.N), prm.device), batch, level,
                            _dev_ptr(out, "d", (batch, 3, level, prm.N), prm.device), _stream()), "pc_tensor")
    return out


def rescale(prm: Params, ct, level: int, out=None):
    """Divide by the last prime, rounded (pc_rescale): [batch][2][level][N] -> [batch][2][level-1][N]."""
    ct = _batched(ct)
    batch = int(ct.shape[0])
    if out is None:
        out = _new((batch, 2, level - 1, prm.N), prm.device)
    _check(_lib().pc_rescale(prm.handle, _dev_ptr(ct, "ct", (batch, 2, level, prm.N), prm.device), batch, level,
                             _dev_ptr(out, "out", (batch, 2, level - 1, prm.N), prm.device), _stream()),
           "pc_rescale")
    return out


def hmult(prm: Params, ct_a, ct_b, evk_b, seed: bytes, level: int, out=None):
    """Tensor, relinearise with the key of s^2 (b half evk_b, a half from seed), rescale (pc_hmult).

    ct_a, ct_b: [batch][2][level][N]; returns [batch][2][level-1][N].
    """
    ct_a, ct_b = _batched(ct_a), _batched(ct_b)
    batch = int(ct_a.shape[0])
    if out is None:
        out = _new((batch, 2, level - 1, prm.N), prm.device)
    _check(_lib().pc_hmult(prm.handle, _dev_ptr(ct_a, "ct_a", (batch, 2, level, prm.N), prm.device),
                           _dev_ptr(ct_b, "ct_b", (batch, 2, level, prm.N), prm.device), batch,
                           _dev_ptr(evk_b, "evk_b", prm.key_shape(level), prm.device), _seed_bytes(seed), level,
                           _dev_ptr(out, "out", (batch, 2, level - 1, prm.N), prm.device), _stream()), "pc_hmult")
    return out


def linear_transform(prm: Params, ct, diag, level: int, baby_b: Sequence = (), baby_seeds: Sequence = (),
                     baby_galois: Sequence[int] = (), giant_b: Sequence = (), giant_seeds: Sequence = (),
                     giant_galois: Sequence[int] = (), out=None):
    """Double-hoisted BSGS linear transform of ct [2][level][N] (pc_linear_transform).

    diag: [n2][n1][level+K][N] plaintext diagonals over the extended basis, with
    n1 = 1 + len(baby keys) and n2 = 1 + len(giant keys); keys are b halves
    (shape prm.key_shape(level)) with 32-byte seeds and Galois elements.
    Returns out [2][level][N].
    """
    n2, n1 = int(diag.shape[0]), int(diag.shape[1])
    if len(baby_b) != n1 - 1 or len(baby_seeds) != n1 - 1 or len(baby_galois) != n1 - 1:
        raise ValueError("diag's second axis must be 1 + the number of baby keys (b, seed, Galois element each)")
    if len(giant_b) != n2 - 1 or len(giant_seeds) != n2 - 1 or len(giant_galois) != n2 - 1:
        raise ValueError("diag's first axis must be 1 + the number of giant keys (b, seed, Galois element each)")
    kshape = prm.key_shape(level)
    lk = level + prm.K
    if out is None:
        out = _new((2, level, prm.N), prm.device)
    args = _LtArgs()
    args.ct = _dev_ptr(ct, "ct", (2, level, prm.N), prm.device)
    args.level = level
    args.n1 = n1
    args.n2 = n2
    args.diag = _dev_ptr(diag, "diag", (n2, n1, lk, prm.N), prm.device)
    keep = []

    def keys(bs, seeds, galois, name):
        n = len(bs)
        if n == 0:
            return None, None, None
        ptrs = (ctypes.c_void_p * n)(*[_dev_ptr(b, name, kshape, prm.device).value for b in bs])
        blob = b"".join(_seed_bytes(x) for x in seeds)
        gal = (ctypes.c_uint32 * n)(*[int(g) for g in galois])
        keep.extend([ptrs, blob, gal])
        return ptrs, blob, gal

    args.baby_b, args.baby_seeds, args.baby_galois = keys(baby_b, baby_seeds, baby_galois, "baby_b")
    args.giant_b, args.giant_seeds, args.giant_galois = keys(giant_b, giant_seeds, giant_galois, "giant_b")
    args.out = _dev_ptr(out, "out", (2, level, prm.N), prm.device)
    _check(_lib().pc_linear_transform(prm.handle, ctypes.byref(args), _stream()), "pc_linear_transform")
    return out


class KeySet:
    """A key bundle (pc_keyset_create): nkeys keys of the key level serving
    ``level``, each its b half plus a 32-byte seed (``full=True`` also stores
    the expanded a halves), in one device allocation."""

    def __init__(self, prm: Params, level: int, galois: Sequence[int], full: bool = False):
        n = len(galois)
        gal = (ctypes.c_uint32 * n)(*[int(g) for g in galois])
        h = ctypes.c_void_p()
        _check(_lib().pc_keyset_create(prm.handle, level, n, gal, PC_KEYSET_FULL if full else PC_KEYSET_PACKED,
                                       ctypes.byref(h)), "pc_keyset_create")
        self._h, self.prm, self.level, self.galois, self.full = h, prm, level, list(galois), full

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("key set closed")
        return self._h

    def close(self):
        if getattr(self, "_h", None) is not None:
            _lib().pc_keyset_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def _get_u64(self, what: int, arg: int = 0) -> int:
        buf = ctypes.c_uint64()
        _check(_lib().pc_keyset_get(self.handle, what, arg, ctypes.byref(buf), 8), "pc_keyset_get")
        return int(buf.value)

    def device_bytes(self) -> int:
        return self._get_u64(PC_KEYSET_DEVICE_BYTES)

    def key_bytes(self) -> int:
        return self._get_u64(PC_KEYSET_KEY_BYTES)

    def set(self, idx: int, evk_b, seed: bytes):
        """Store key idx: its b half (device, the key shape) and its seed (pc_keyset_set)."""
        ptr = _dev_ptr(evk_b, "evk_b", self.prm.key_shape(self.level), self.prm.device)
        _check(_lib().pc_keyset_set(self.handle, idx, ptr, _seed_bytes(seed), _stream()), "pc_keyset_set")

    def keygen(self, idx: int, seed: bytes, s_coef, e_coef):
        """Generate key idx in place (pc_keyset_keygen); s_coef, e_coef as in keygen()."""
        kl = self.prm.key_level(self.level)
        lk = kl + self.prm.K
        beta = self.prm.beta(kl)
        _check(_lib().pc_keyset_keygen(self.handle, idx, _seed_bytes(seed),
                                       _dev_ptr(s_coef, "s_coef", (lk, self.prm.N), self.prm.device),
                                       _dev_ptr(e_coef, "e_coef", (beta, lk, self.prm.N), self.prm.device),
                                       _stream()), "pc_keyset_keygen")


def keyswitch_keyset(prm: Params, keyset: KeySet, ct, key_idx: Sequence[int], level: int, out=None, workspace=None):
    """ct [batch][2][level][N] under the bundle's keys key_idx (pc_keyswitch_keyset);
    returns out [len(key_idx)][batch][2][level][N]."""
    batch, nsel = int(ct.shape[0]), len(key_idx)
    if out is None:
        out = _new((nsel, batch, 2, level, prm.N), prm.device)
    idx = (ctypes.c_uint32 * nsel)(*[int(i) for i in key_idx])
    ws, ws_bytes = None, 0
    if workspace is not None:
        ws = _dev_ptr(workspace, "workspace", None, prm.device)
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib().pc_keyswitch_keyset(prm.handle, keyset.handle, _dev_ptr(ct, "ct", (batch, 2, level, prm.N),
                                                                           prm.device),
                                      batch, idx, nsel, level,
                                      _dev_ptr(out, "out", (nsel, batch, 2, level, prm.N), prm.device), ws,
                                      ws_bytes, _stream()), "pc_keyswitch_keyset")
    return out


def chacha_expand(prm: Params, seed: bytes, d: int, j: int, level: int, out=None):
    """Limb j (key basis at level) of digit d of the regenerated a half (pc_chacha_expand)."""
    if out is None:
        out = _new((prm.N,), prm.device)
    _check(_lib().pc_chacha_expand(prm.handle, _seed_bytes(seed), d, j, level,
                                   _dev_ptr(out, "out", (prm.N,), prm.device), _stream()), "pc_chacha_expand")
    return out


def profile_begin(prm: Params):
    """Start bracketing every kernel launch of ``prm`` with HIP events (pc_profile_begin)."""
    _check(_lib().pc_profile_begin(prm.handle), "pc_profile_begin")


def profile_end(prm: Params) -> dict:
    """Stop and return {kernel family: (launches, summed milliseconds)} (pc_profile_end)."""
    stats = (_KStat * 32)()
    n = ctypes.c_uint32()
    _check(_lib().pc_profile_end(prm.handle, stats, 32, ctypes.byref(n)), "pc_profile_end")
    return {stats[i].name.decode(): (int(stats[i].launches), float(stats[i].total_ms)) for i in range(n.value)}


# host <-> device helpers (uint32 residues held in int32 tensors)
def to_device(arr, device: int = 0):
    import numpy as np
    import torch
    a = np.ascontiguousarray(np.asarray(arr).astype(np.uint32)).view(np.int32)
    return torch.from_numpy(a).to(f"cuda:{device}")


def to_host(t):
    import numpy as np
    return t.detach().cpu().numpy().view(np.uint32)
