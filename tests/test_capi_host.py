"""The C-ABI library on the CPU: loading, exported symbols, host tables, validation.

No compute call reaches a GPU here: parameters are created host-only
(device = -1) and every compute entry point must reject its arguments, or
report PC_EDEVICE, before touching HIP.
"""

import ctypes
import json
import os
import re

import pytest

import key_switching_amd as ksa
from oracle import keyswitch as ks
from oracle import rns

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")

pytestmark = pytest.mark.skipif(not os.path.exists(ksa.LIB_PATH), reason="libpc.so not built")


def declared_functions():
    text = open(os.path.join(ROOT, "include", "pc.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(pc_\w+)\s*\(", text))


def test_exports_every_declared_symbol():
    declared = declared_functions()
    assert declared == set(ksa.EXPORTED)
    lib = ctypes.CDLL(ksa.LIB_PATH)
    for name in declared:
        assert getattr(lib, name) is not None


@pytest.mark.parametrize("log2n,L,dnum,K", [(12, 3, 3, 1), (16, 24, 4, 6), (17, 40, 5, 8)])
def test_host_tables_match_golden(log2n, L, dnum, K):
    with ksa.Params(log2n, L, dnum, K, device=None) as prm:
        g = json.load(open(os.path.join(GOLDEN, f"chain_n{log2n}.json")))
        assert prm.primes == g["primes"][: L + K]
        assert prm.psi == g["psi"][: L + K]
        N = 1 << log2n
        for pi in (0, L + K - 1):
            tw = prm.twiddles(pi)
            q, psi = g["primes"][pi], g["psi"][pi]
            for k in (0, 1, 2, 3, N // 2, N - 1):
                e = int(format(k, f"0{log2n}b")[::-1], 2)
                assert tw[k] == pow(psi, e, q)


@pytest.mark.parametrize("partition", [0, 1])
@pytest.mark.parametrize("L,dnum", [(24, 4), (40, 5), (3, 3), (7, 3), (6, 6)])
def test_digit_partition_matches_oracle(L, dnum, partition):
    with ksa.Params(12, L, dnum, 2, device=None, partition=partition) as prm:
        oprm = ks.Params(12, L, dnum, 2, primes=tuple(prm.primes), partition=partition)
        for level in range(1, L + 1):
            D = oprm.digits(level)
            assert prm.beta(level) == len(D)
            assert prm.alpha(level) == oprm.alpha(level)
            assert len(D[0]) == min(oprm.alpha(level), level)
            assert prm.key_level(level) == oprm.key_level(level)
            assert prm.key_shape(level) == (len(oprm.digits(oprm.key_level(level))), oprm.key_level(level) + 2,
                                            oprm.N)


def test_user_primes_accepted_and_checked():
    N = 1 << 12
    chain = rns.ntt_primes(N, 6)[2:]
    with ksa.Params(12, 3, 1, 1, primes=chain, device=None) as prm:
        assert prm.primes == chain
    bad = [chain[0], chain[1], chain[2], chain[3] + 2 * N]  # not prime or not 1 mod 2N
    for b in (bad, [chain[0]] * 4, [97, 193, 257, 449]):
        with pytest.raises(ksa.PcError) as e:
            ksa.Params(12, 3, 1, 1, primes=b, device=None)
        assert e.value.code == ksa.PC_EINVAL


@pytest.mark.parametrize("kw,code", [
    (dict(log2n=13, L=3, dnum=3, K=1), ksa.PC_EUNSUPPORTED),
    (dict(log2n=12, L=3, dnum=4, K=1), ksa.PC_EINVAL),
    (dict(log2n=12, L=0, dnum=1, K=1), ksa.PC_EINVAL),
    (dict(log2n=12, L=3, dnum=3, K=0), ksa.PC_EINVAL),
    (dict(log2n=12, L=8, dnum=7, K=1), ksa.PC_EUNSUPPORTED),
    (dict(log2n=12, L=3, dnum=3, K=1, chacha_rounds=8), ksa.PC_EUNSUPPORTED),
    (dict(log2n=12, L=3, dnum=3, K=1, max_hoist=33), ksa.PC_EUNSUPPORTED),
    (dict(log2n=12, L=3, dnum=3, K=9), ksa.PC_EUNSUPPORTED),
    (dict(log2n=16, L=24, dnum=2, K=6), ksa.PC_EUNSUPPORTED),
    (dict(log2n=12, L=3, dnum=3, K=1, partition=2), ksa.PC_EINVAL),
])
def test_create_rejects(kw, code):
    with pytest.raises(ksa.PcError) as e:
        ksa.Params(device=None, **kw)
    assert e.value.code == code


def test_compute_calls_validate_before_touching_a_device():
    lib = ksa._lib()
    with ksa.Params(12, 3, 3, 1, device=None) as prm:
        h = prm.handle
        dummy = ctypes.c_void_p(0x1000)  # never dereferenced: validation or the device check fails first
        idx = (ctypes.c_uint32 * 1)(0)
        bad_idx = (ctypes.c_uint32 * 1)(4)
        assert lib.pc_ntt(h, None, idx, 1, 1, None) == ksa.PC_EINVAL
        assert lib.pc_ntt(h, dummy, bad_idx, 1, 1, None) == ksa.PC_EINVAL
        assert lib.pc_ntt(h, dummy, idx, 1, 1, None) == ksa.PC_EDEVICE
        assert lib.pc_intt(h, dummy, idx, 1, 3, None) == ksa.PC_EDEVICE
        assert lib.pc_modup(h, dummy, 0, dummy, None) == ksa.PC_EINVAL
        assert lib.pc_modup(h, dummy, 4, dummy, None) == ksa.PC_EINVAL
        assert lib.pc_modup(h, dummy, 3, dummy, None) == ksa.PC_EDEVICE
        assert lib.pc_moddown(h, dummy, 3, None, None) == ksa.PC_EINVAL
        seed = bytes(32)
        assert lib.pc_keyswitch(h, dummy, dummy, seed, 3, 4, dummy, None) == ksa.PC_EINVAL  # even Galois element
        assert lib.pc_keyswitch(h, dummy, dummy, seed, 3, 1 << 13, dummy, None) == ksa.PC_EINVAL
        assert lib.pc_keyswitch(h, dummy, dummy, None, 3, 5, dummy, None) == ksa.PC_EINVAL
        assert lib.pc_keyswitch(h, dummy, dummy, seed, 9, 5, dummy, None) == ksa.PC_EINVAL
        assert lib.pc_keyswitch(h, dummy, dummy, seed, 3, 5, dummy, None) == ksa.PC_EDEVICE
        assert lib.pc_chacha_expand(h, seed, 3, 0, 3, dummy, None) == ksa.PC_EINVAL  # beta = 3 digits
        assert lib.pc_chacha_expand(h, seed, 0, 4, 3, dummy, None) == ksa.PC_EINVAL  # 3 + K limbs
        assert lib.pc_chacha_expand(h, seed, 2, 3, 3, dummy, None) == ksa.PC_EDEVICE
        # batch above max_batch
        args = ksa._KsArgs()
        args.ct, args.batch, args.nkeys, args.level, args.out = dummy, 2, 1, 3, dummy
        bp = (ctypes.c_void_p * 1)(0x1000)
        gal = (ctypes.c_uint32 * 1)(5)
        args.evk_b, args.galois, args.seeds = bp, gal, seed
        assert lib.pc_keyswitch_ex(h, ctypes.byref(args), None) == ksa.PC_EINVAL
        args.batch = 1
        assert lib.pc_keyswitch_ex(h, ctypes.byref(args), None) == ksa.PC_EDEVICE
        args.seeds = None
        assert lib.pc_keyswitch_ex(h, ctypes.byref(args), None) == ksa.PC_EINVAL
        # pc_keygen: arguments first, then the device
        assert lib.pc_keygen(h, None, 3, 1, dummy, dummy, dummy, None) == ksa.PC_EINVAL
        assert lib.pc_keygen(h, seed, 3, 1, None, dummy, dummy, None) == ksa.PC_EINVAL
        assert lib.pc_keygen(h, seed, 4, 1, dummy, dummy, dummy, None) == ksa.PC_EINVAL
        assert lib.pc_keygen(h, seed, 3, 6, dummy, dummy, dummy, None) == ksa.PC_EINVAL
        assert lib.pc_keygen(h, seed, 3, 5, dummy, dummy, dummy, None) == ksa.PC_EDEVICE
        # pc_tensor / pc_rescale / pc_hmult (max_batch 1, L 3)
        assert lib.pc_tensor(h, None, dummy, 1, 3, dummy, None) == ksa.PC_EINVAL
        assert lib.pc_tensor(h, dummy, dummy, 0, 3, dummy, None) == ksa.PC_EINVAL
        assert lib.pc_tensor(h, dummy, dummy, 2, 3, dummy, None) == ksa.PC_EINVAL
        assert lib.pc_tensor(h, dummy, dummy, 1, 4, dummy, None) == ksa.PC_EINVAL
        assert lib.pc_tensor(h, dummy, dummy, 1, 3, dummy, None) == ksa.PC_EDEVICE
        assert lib.pc_rescale(h, dummy, 1, 1, dummy, None) == ksa.PC_EINVAL  # nothing left to drop to
        assert lib.pc_rescale(h, dummy, 1, 4, dummy, None) == ksa.PC_EINVAL
        assert lib.pc_rescale(h, dummy, 1, 3, None, None) == ksa.PC_EINVAL
        assert lib.pc_rescale(h, dummy, 1, 2, dummy, None) == ksa.PC_EDEVICE
        assert lib.pc_hmult(h, dummy, dummy, 1, dummy, None, 3, dummy, None) == ksa.PC_EINVAL
        assert lib.pc_hmult(h, dummy, dummy, 1, dummy, seed, 1, dummy, None) == ksa.PC_EINVAL
        assert lib.pc_hmult(h, dummy, dummy, 2, dummy, seed, 3, dummy, None) == ksa.PC_EINVAL
        assert lib.pc_hmult(h, dummy, None, 1, dummy, seed, 3, dummy, None) == ksa.PC_EINVAL
        assert lib.pc_hmult(h, dummy, dummy, 1, dummy, seed, 3, dummy, None) == ksa.PC_EDEVICE
        # pc_linear_transform: sizes, keys, then the device
        lt = ksa._LtArgs()
        lt.ct, lt.diag, lt.out, lt.level, lt.n1, lt.n2 = dummy.value, dummy.value, dummy.value, 3, 1, 1
        assert lib.pc_linear_transform(h, None, None) == ksa.PC_EINVAL
        assert lib.pc_linear_transform(h, ctypes.byref(lt), None) == ksa.PC_EDEVICE
        for field, bad in (("n1", 0), ("n1", 9), ("n2", 0), ("n2", 33), ("level", 0), ("level", 4)):
            good = getattr(lt, field)
            setattr(lt, field, bad)
            assert lib.pc_linear_transform(h, ctypes.byref(lt), None) == ksa.PC_EINVAL, (field, bad)
            setattr(lt, field, good)
        lt.n1 = 2  # one baby key is now required
        assert lib.pc_linear_transform(h, ctypes.byref(lt), None) == ksa.PC_EINVAL
        ptrs = (ctypes.c_void_p * 1)(dummy.value)
        gal = (ctypes.c_uint32 * 1)(4)
        lt.baby_b, lt.baby_seeds, lt.baby_galois = ptrs, seed, gal
        assert lib.pc_linear_transform(h, ctypes.byref(lt), None) == ksa.PC_EINVAL  # even Galois element
        gal[0] = 5
        assert lib.pc_linear_transform(h, ctypes.byref(lt), None) == ksa.PC_EDEVICE
        lt.ct = None
        assert lib.pc_linear_transform(h, ctypes.byref(lt), None) == ksa.PC_EINVAL
        # params_get argument checks
        buf = (ctypes.c_uint32 * 4)()
        assert lib.pc_params_get(h, ksa.PC_GET_PRIMES, 0, buf, 12) == ksa.PC_EINVAL
        assert lib.pc_params_get(h, ksa.PC_GET_ALPHA, 0, buf, 4) == ksa.PC_EINVAL
        assert lib.pc_params_get(h, 99, 0, buf, 4) == ksa.PC_EINVAL
    assert lib.pc_strerror(ksa.PC_EDEVICE).startswith(b"device")


def test_misaligned_pointers_rejected():
    """The kernels move limbs in 16-byte vectors: a device pointer off a 16-byte
    boundary is refused before anything else (here a host-only params, which
    would otherwise answer PC_EDEVICE)."""
    lib = ksa._lib()
    with ksa.Params(12, 3, 3, 1, device=None, max_batch=2) as prm:
        h = prm.handle
        ok, bad = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1004)
        idx = (ctypes.c_uint32 * 1)(0)
        seed = bytes(32)
        assert lib.pc_ntt(h, bad, idx, 1, 1, None) == ksa.PC_EINVAL
        assert lib.pc_modup(h, ok, 3, bad, None) == ksa.PC_EINVAL
        assert lib.pc_moddown(h, bad, 3, ok, None) == ksa.PC_EINVAL
        assert lib.pc_keyswitch(h, bad, ok, seed, 3, 5, ok, None) == ksa.PC_EINVAL
        assert lib.pc_keyswitch(h, ok, bad, seed, 3, 5, ok, None) == ksa.PC_EINVAL
        assert lib.pc_keyswitch(h, ok, ok, seed, 3, 5, bad, None) == ksa.PC_EINVAL
        assert lib.pc_keyswitch(h, ok, ok, seed, 3, 5, ok, None) == ksa.PC_EDEVICE
        args = ksa._KsArgs()
        bp = (ctypes.c_void_p * 1)(0x1000)
        gal = (ctypes.c_uint32 * 1)(5)
        args.ct, args.batch, args.nkeys, args.level, args.out = ok, 1, 1, 3, ok
        args.evk_b, args.galois, args.seeds = bp, gal, seed
        args.workspace, args.workspace_bytes = ctypes.c_void_p(0x2008), 1 << 30
        assert lib.pc_keyswitch_ex(h, ctypes.byref(args), None) == ksa.PC_EINVAL
        args.workspace = ctypes.c_void_p(0x2000)
        assert lib.pc_keyswitch_ex(h, ctypes.byref(args), None) == ksa.PC_EDEVICE
        assert lib.pc_keygen(h, seed, 3, 5, ok, bad, ok, None) == ksa.PC_EINVAL
        assert lib.pc_tensor(h, ok, ok, 1, 3, bad, None) == ksa.PC_EINVAL
        assert lib.pc_rescale(h, bad, 1, 3, ok, None) == ksa.PC_EINVAL
        assert lib.pc_hmult(h, ok, ok, 1, bad, seed, 3, ok, None) == ksa.PC_EINVAL
        assert lib.pc_chacha_expand(h, seed, 0, 0, 3, bad, None) == ksa.PC_EINVAL


def test_rescale_and_hmult_launch_limits_checked_on_the_host():
    """A rescale launch carries the constants of at most 256 polynomials: a params
    set whose max_batch allows more is refused with PC_EUNSUPPORTED before any work."""
    lib = ksa._lib()
    with ksa.Params(12, 3, 3, 1, device=None, max_batch=200) as prm:
        h, ok, seed = prm.handle, ctypes.c_void_p(0x1000), bytes(32)
        assert lib.pc_rescale(h, ok, 129, 3, ok, None) == ksa.PC_EUNSUPPORTED
        assert lib.pc_hmult(h, ok, ok, 129, ok, seed, 3, ok, None) == ksa.PC_EUNSUPPORTED
        assert lib.pc_rescale(h, ok, 128, 3, ok, None) == ksa.PC_EDEVICE
        assert lib.pc_hmult(h, ok, ok, 128, ok, seed, 3, ok, None) == ksa.PC_EDEVICE


def test_keyset_calls_validate_before_touching_a_device():
    lib = ksa._lib()
    with ksa.Params(12, 3, 3, 1, device=None) as prm:
        h = prm.handle
        out = ctypes.c_void_p()
        gal = (ctypes.c_uint32 * 3)(5, 25, 1)
        assert lib.pc_keyset_create(h, 3, 3, gal, 0, ctypes.byref(out)) == ksa.PC_EDEVICE
        assert lib.pc_keyset_create(h, 3, 3, gal, 2, ctypes.byref(out)) == ksa.PC_EINVAL
        assert lib.pc_keyset_create(h, 4, 3, gal, 0, ctypes.byref(out)) == ksa.PC_EINVAL
        assert lib.pc_keyset_create(h, 3, 0, gal, 0, ctypes.byref(out)) == ksa.PC_EINVAL
        dup = (ctypes.c_uint32 * 2)(5, 5)
        assert lib.pc_keyset_create(h, 3, 2, dup, 0, ctypes.byref(out)) == ksa.PC_EINVAL
        even = (ctypes.c_uint32 * 1)(4)
        assert lib.pc_keyset_create(h, 3, 1, even, 0, ctypes.byref(out)) == ksa.PC_EINVAL
        assert lib.pc_keyset_create(None, 3, 1, gal, 0, ctypes.byref(out)) == ksa.PC_EINVAL
        assert out.value is None
        assert lib.pc_keyset_set(None, 0, ctypes.c_void_p(0x1000), bytes(32), None) == ksa.PC_EINVAL
        idx = (ctypes.c_uint32 * 1)(0)
        assert lib.pc_keyswitch_keyset(h, None, ctypes.c_void_p(0x1000), 1, idx, 1, 3, ctypes.c_void_p(0x1000),
                                       None, 0, None) == ksa.PC_EINVAL


def test_every_declaration_cites_the_pages():
    """Each entry point's comment in include/pc.h names the page and section that
    defines the operation (the error-text helper excepted: no page defines it;
    the allocation-free variant of the key switch names the callers it serves
    instead)."""
    text = open(os.path.join(ROOT, "include", "pc.h")).read()
    blocks = [(m.end(), m.group(0)) for m in re.finditer(r"^/\*.*?\*/", text, flags=re.M | re.S)]
    code = re.sub(r"/\*.*?\*/", lambda m: " " * len(m.group(0)), text, flags=re.S)
    def comment_of(name):
        pos = code.index(name + "(")
        before = [b for end, b in blocks if end <= pos]
        assert before, name
        return before[-1]

    if "pc_keyswitch_static" in declared_functions():
        assert "cannot allocate" in comment_of("pc_keyswitch_static")
    for name in sorted(declared_functions() - {"pc_strerror", "pc_keyswitch_static"}):
        comment = comment_of(name)
        assert "Perseus README" in comment or "arXiv summary page" in comment, name
        assert re.search(r"'[A-Z][^']*'", comment), f"{name}: no section named"


def test_arena_and_transform_workspace_sizes():
    with ksa.Params(16, 24, 4, 6, max_batch=8, device=None) as prm:
        arena = prm.arena_bytes()
        assert arena >= prm.workspace_bytes(24)
        need = prm.lt_workspace_bytes(24, 4, 4)
        assert 0 < need <= arena  # the 4 x 4 transform fits the batch-8 arena
        assert prm.lt_workspace_bytes(24, 8, 4) > need and prm.lt_workspace_bytes(24, 4, 8) > need
        assert prm.lt_workspace_bytes(12, 4, 4) < need
    with ksa.Params(16, 24, 4, 6, device=None) as small:
        assert small.lt_workspace_bytes(24, 4, 4) > small.arena_bytes()  # needs a larger arena
        with pytest.raises(ksa.PcError):
            small.lt_workspace_bytes(25, 4, 4)


def test_workspace_grows_with_level():
    with ksa.Params(16, 24, 4, 6, max_batch=8, device=None) as prm:
        sizes = [prm.workspace_bytes(l) for l in (4, 8, 12, 16, 20, 24)]
        assert sizes == sorted(sizes) and sizes[0] > 0


def test_arena_fits_every_level():
    """With ceil(l/dnum) primes per digit a lower level can need a larger
    workspace than the top one (more digits): L = 6, dnum = 5 has 3 digits at
    level 6 and 5 at level 5. The arena covers every level."""
    prm = ksa.Params(12, 6, 5, 2, device=None, max_batch=1, max_hoist=2)
    sizes = [prm.workspace_bytes(level) for level in range(1, 7)]
    assert max(sizes) > sizes[-1]
    assert prm.arena_bytes() >= max(sizes)
    prm.close()
