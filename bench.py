#!/usr/bin/env python3
"""Throughput of CKKS hybrid key switching on one MI355X.

A step is one call of the whole hot path (ModUp, automorphism + inner product
with the ChaCha12-regenerated key half, ModDown) on one batch of synthetic
ciphertexts at N=2^16, L=24, dnum=4, K=6 with one relinearisation key: the
workload the headline metric (key switches/s at N=2^16, L=24, k=1 and 8) is
quoted on. `value` is key switches per second at batch k=8; the k=1 rate and
the stored-key variants are reported beside it.

The headline runs the batches one after another on one HIP stream: with the
clock up, a batch of 8 fills the chip and one stream measured faster than two
or three (0.47-0.49 against 0.50-0.53 ms per batch). Independent calls dealt round-robin to
several streams (`--streams`, each call with its own caller workspace) are
reported beside it; at batch 1 they overlap calls that each leave most of the
chip idle.

Inputs are resident in HBM before timing starts. Ciphertext inputs and outputs
rotate through more than 1 GiB of buffers so that the 256 MB Infinity Cache
cannot hold them between steps; the key is reused, as in real
relinearisation. The key's b half is a uniform draw (a real b half is
indistinguishable from uniform) so that timing never depends on key
generation.

Beside the headline the line carries per-step min/median/max, a measured
stream-copy bandwidth (context for the 8 TB/s peak), the homomorphic
multiplication, linear-transform and key-generation legs, and the key-switch
rates of the other workloads (one ciphertext under 16 hoisted rotation keys,
the level sweep 24..4, the N=2^17 relinearise-then-rotate chain).

Prints one JSON line. `python bench.py --gpus N` with N > 1 exits: the
benchmark measures one GPU.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import ks_inputs as ki  # noqa: E402

METRIC = "key switches/sec at N=2^16, L=24 (k=1,8); % of HBM/INT32 roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
CUS, CLOCK_GHZ = 256, 2.4       # MI355X compute units and peak engine clock
INT32_LANES_PER_CU = 64         # 4 SIMDs x 16 lanes; every 32-bit integer VALU op issues at this rate
INT32_PEAK_TOPS = CUS * INT32_LANES_PER_CU * CLOCK_GHZ / 1000.0  # 39.3 T int32 lane-ops/s

# 32-bit integer operations of the arithmetic primitives (the minimum instruction
# count of each with canonical residues below r < 2^31):
OPS_MONT = 5        # x*w 2^-32 mod r: 64-bit product, m = lo*(-r^-1), + m*r, high word, one correction
OPS_ADDMOD = 3      # add, subtract r, unsigned min
OPS_BUTTERFLY = OPS_MONT + 2 * OPS_ADDMOD   # one twiddle product, one modular add, one modular subtract
OPS_SHOUP = 5       # multiply by a constant with its Shoup companion
OPS_REDC = 4        # low word times -r^-1, multiply-add, subtract r, min
OPS_CHACHA12_BLOCK = 6 * 8 * 12 + 16        # 6 double rounds x 8 quarter rounds x 12 ops, + feed-forward
OPS_WORDPAIR = 6 + OPS_REDC                 # two words -> a residue in Montgomery form


def dot_ops(alpha):
    """Base-conversion dot product of alpha sources: one multiply-add each, a fold of
    the 64-bit sum after the fourth product and every further pair (two ops each), REDC."""
    folds = 0 if alpha <= 2 else 1 + (alpha - 3) // 2
    return alpha + 2 * folds + OPS_REDC


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--spinup-ms", type=float, default=300.0,
                    help="untimed batch-8 key switches (about this much GPU time) before the first timed leg and "
                         "before the multi-stream legs, so that every leg runs at the clock of a loaded GPU")
    ap.add_argument("--long-steps", type=int, default=2000,
                    help="steps of the steady-state leg (batch 8, one stream, ~1 s of GPU time)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="per-leg budget of the oracle baseline (one thread, then every thread)")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="OpenMP threads of the all-core oracle leg (0: this process's CPU share, at most 16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--buffers-gib", type=float, default=1.1, help="ciphertext buffer rotation size")
    ap.add_argument("--streams", type=int, default=3, choices=(1, 2, 3),
                    help="streams of the labelled variants with independent calls in flight (each call with "
                         "its own workspace; the headline is one stream); 1 skips them, as profiler runs "
                         "need, whose per-dispatch times must not overlap")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the timings of the other workloads (hoisted 16, level sweep, N=2^17 chain)")
    ap.add_argument("--only", choices=("hoist16", "levels16", "n17"), default=None,
                    help="time only this workload (regenerated and stored key halves), for profiler runs")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 256 MiB copy kernel (reference for rocprofv3 byte counters)")
    return ap.parse_args()


LRC = {12: 6, 16: 8, 17: 8}   # NTT stages in the column pass (the block pass does the rest)


def _shape(N, level, K, alpha, beta):
    digits = [min(alpha, level - d * alpha) for d in range(beta)]
    lrc = LRC[N.bit_length() - 1]
    return digits, sum(level + K - a for a in digits), lrc, N.bit_length() - 1 - lrc


def alg_bytes(kernel, N, level, K, alpha, beta, batch, nkeys=1, stored=False):
    """Algorithmic bytes one launch must move: each input limb read once, each output limb written once.

    Limb = N words of 4 bytes; T_d = level - alpha_d + K targets per digit; the
    inner product reads each key's b half (and with ``stored`` its a half) once
    per batch; ModDown runs on 2 polynomials of every (key, ciphertext) item.
    """
    l, limb = level, 4 * N
    _, targets, _, _ = _shape(N, level, K, alpha, beta)
    items = batch * nkeys
    table = {
        # ModUp: c1 in, y' out; y' in place (scaled y); y in, targets out; targets in, ext out
        "modup_inv_blk": batch * (l + l),
        "modup_inv_col": batch * (l + l),
        "modup_bconv": batch * (l + targets),
        "modup_fwd_blk": batch * (targets + targets),
        # IP: ext (targets) + own c1 limbs read once per key, b read once per key, acc written
        "inner_product": nkeys * (batch * (targets + l) + (2 if stored else 1) * beta * (l + K))
                         + items * 2 * (l + K),
        "moddown_inv_blk": items * 2 * (K + K),
        "moddown_inv_col": items * 2 * (K + K),
        "moddown_bconv": items * 2 * (K + l),
        "moddown_fwd_blk": items * 2 * (l + l + l) + items * l,  # tmp2 + acc in, out; c0 in
    }
    # the fused block pass and inner product (one key of Galois element 1): the
    # column-pass output and c1's own limbs in, the key once, acc out
    table["modup_ip"] = (batch * (targets + l) + (2 if stored else 1) * beta * (l + K)) + items * 2 * (l + K)
    return table[kernel] * limb


def alg_ops(kernel, N, level, K, alpha, beta, batch, nkeys=1, stored=False):
    """Algorithmic 32-bit integer operations of one launch (op counts of the primitives above).

    An NTT pass over a limb does N/2 butterflies per stage: the column pass
    covers the first LRC stages, the block pass the rest. With ``stored`` the
    key's a half is read and put in Montgomery form instead of regenerated.
    """
    l = level
    digits, targets, lrc, lrb = _shape(N, level, K, alpha, beta)
    col = N // 2 * lrc * OPS_BUTTERFLY
    blk = N // 2 * lrb * OPS_BUTTERFLY
    conv_targets = sum((l + K - a) * N * dot_ops(a) for a in digits)
    lk = l + K
    items = batch * nkeys
    a_ops = OPS_REDC if stored else OPS_CHACHA12_BLOCK / 8 + OPS_WORDPAIR
    key_ops = lk * N * beta * (OPS_REDC + a_ops)  # b to Montgomery form, a regenerated (or read)
    ip_item = lk * N * 2 * dot_ops(beta)                                            # both sums, one REDC each
    table = {
        "modup_inv_blk": batch * l * blk,
        "modup_inv_col": batch * l * (col + N * OPS_SHOUP),
        "modup_bconv": batch * (conv_targets + targets * col),
        "modup_fwd_blk": batch * targets * blk,
        "inner_product": nkeys * key_ops + items * ip_item,
        "moddown_inv_blk": items * 2 * K * blk,
        "moddown_inv_col": items * 2 * K * (col + N * OPS_SHOUP),
        "moddown_bconv": items * 2 * l * (N * dot_ops(K) + col),
        "moddown_fwd_blk": items * 2 * l * (blk + N * (2 * OPS_ADDMOD + OPS_SHOUP)),
    }
    table["modup_ip"] = table["modup_fwd_blk"] + table["inner_product"]
    return table[kernel]


KERNELS = ("modup_inv_blk", "modup_inv_col", "modup_bconv", "modup_fwd_blk", "inner_product",
           "moddown_inv_blk", "moddown_inv_col", "moddown_bconv", "moddown_fwd_blk")


def alg_bytes_per_launch(kernel, w, batch, beta, alpha):
    return alg_bytes(kernel, w.N, w.L, w.K, alpha, beta, batch)


def alg_ops_per_launch(kernel, w, batch, beta, alpha):
    return alg_ops(kernel, w.N, w.L, w.K, alpha, beta, batch)


def path_fractions(calls, ms, stored=False):
    """HBM and int32-ALU fractions of a measured call made of the key-switch launches in
    `calls` (a list of (N, level, K, alpha, beta, batch, nkeys, with_modup) tuples)."""
    nbytes = nops = 0
    for (N, level, K, alpha, beta, batch, nkeys, with_modup) in calls:
        for k in KERNELS:
            if k.startswith("modup") and not with_modup:
                continue
            nbytes += alg_bytes(k, N, level, K, alpha, beta, batch, nkeys, stored)
            nops += alg_ops(k, N, level, K, alpha, beta, batch, nkeys, stored)
    t = ms * 1e-3
    return {"alg_bytes_per_call": int(nbytes), "alg_ops_per_call": int(nops),
            "hbm_frac": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
            "alu_frac": round(nops / t / 1e12 / INT32_PEAK_TOPS, 4)}


def kernel_roofline(kernel, avg_us, w, batch, beta, alpha):
    """HBM and int32-ALU fractions of one launch; the binding one is the larger."""
    t = avg_us * 1e-6
    nbytes = alg_bytes_per_launch(kernel, w, batch, beta, alpha)
    nops = alg_ops_per_launch(kernel, w, batch, beta, alpha)
    hbm = nbytes / t / 1e9
    alu = nops / t / 1e12
    return {"hbm_gbs": round(hbm, 1), "hbm_frac": round(hbm / HBM_PEAK_GBS, 4),
            "alu_tops": round(alu, 2), "alu_frac": round(alu / INT32_PEAK_TOPS, 4),
            "alg_bytes": nbytes, "alg_ops": int(nops), "avg_us": round(avg_us, 3)}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_share():
    """Cores this process may use: its affinity set, capped by the thread budget the
    environment sets (OMP_NUM_THREADS) and by 16."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    try:
        env = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        env = 0
    if env > 0:
        n = min(n, env)
    return max(1, min(n, 16))


def _o2_sample(O, w, ct, b, seed, threads, budget_s, max_calls=400):
    """Key switches by the C++ oracle until the budget is used: (calls, seconds)."""
    n, t0 = 0, time.perf_counter()
    while True:
        O.keyswitch(ct[n % len(ct)], w.L, 1, b, seed=seed, threads=threads, validate=False)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= max_calls:
            return n, el


def _numpy_oracle_one_core(w, calls=2):
    """The numpy oracle on one core, a few calls (context for the C++ figure)."""
    from oracle import keyswitch as ks
    oprm = ks.Params(w.log2n, w.L, w.dnum, w.K)
    beta = len(oprm.digits(w.L))
    key = ks.Key(b=ki.uniform_key_b(w.index, 0, beta, oprm.basis(w.L), w.N), seed=ki.key_seed(w.index, 0),
                 level=w.L, galois=1)
    cts = ki.ciphertexts(w.index, oprm.q, w.N, calls)
    ks.keyswitch(oprm, cts[0], key, w.L)  # fills the oracle's table caches (not timed)
    t0 = time.perf_counter()
    for c in cts:
        ks.keyswitch(oprm, c, key, w.L)
    return calls / (time.perf_counter() - t0)


def cpu_baseline(w, budget_s, threads):
    """The C++ oracle tier as it stands (oracle/ks_o2.cpp: plain C++, every product a 64-bit
    `%`, OpenMP over independent (digit, limb) items) on a bounded sample of the headline
    workload: single-ciphertext N=2^16, L=24 key switches with the workload's key shape and a
    ChaCha12-regenerated a half, first on one thread, then on `threads` threads, each leg until
    its budget is used (at most 400 calls); then the numpy oracle on one core for two calls.
    The clock brackets the key-switch calls only. Rate = key switches per second."""
    from oracle import o2
    O = o2.O2(w.log2n, w.L, w.dnum, w.K)
    basis = O.primes[: w.L] + O.primes[w.L:]
    alpha = -(-w.L // w.dnum)
    beta = -(-w.L // alpha)
    b = np.ascontiguousarray(ki.uniform_key_b(w.index, 0, beta, basis, w.N), dtype=np.uint32)
    seed = ki.key_seed(w.index, 0)
    ct = [np.ascontiguousarray(x, dtype=np.uint32) for x in ki.ciphertexts(w.index, O.primes[: w.L], w.N, 4)]
    O.keyswitch(ct[0], w.L, 1, b, seed=seed, threads=threads)  # checks the inputs once (not timed)
    n1, t1 = _o2_sample(O, w, ct, b, seed, 1, budget_s)
    nall, tall = _o2_sample(O, w, ct, b, seed, threads, budget_s) if threads > 1 else (n1, t1)
    O.close()
    one, allc = n1 / t1, nall / tall
    numpy_one = _numpy_oracle_one_core(w)
    return {"value": round(allc, 4), "unit": "key switches/s", "cores": threads, "kind": "oracle",
            "sample": (f"{nall} single-ciphertext key switches (N=2^16, L=24, dnum=4, K=6, ChaCha12 a half) by the "
                       f"C++ oracle tier on {threads} OpenMP threads in {tall:.1f} s; one thread: {n1} in {t1:.1f} s"),
            "one_core_value": round(one, 4), "numpy_oracle_one_core_value": round(numpy_one, 4),
            "cpu_model": _cpu_model(), "host_cpu_count": os.cpu_count()}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(key switching shards by ciphertext batch; see the design notes).", file=sys.stderr)
        sys.exit(2)
    w = ki.WORKLOADS["n16"]
    # the oracle baseline runs first, before the GPU is touched
    cpu = None
    if not args.no_cpu_baseline and args.only is None:
        cpu = cpu_baseline(w, args.cpu_seconds, args.cpu_threads or _cpu_share())
        print(f"[bench] cpu baseline: {cpu['value']} ks/s on {cpu['cores']} cores, {cpu['one_core_value']} on one",
              file=sys.stderr, flush=True)

    import torch
    import key_switching_amd as ksa

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.ones(64 << 20, dtype=torch.int32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.bitwise_or(src, 0, out=dst)
        del src, dst
        torch.cuda.synchronize()
    if args.only is not None:
        res = other_configs(ksa, torch, args, only=args.only)
        print(json.dumps({"only": args.only, "other_configs": res}), flush=True)
        return
    K8 = 8
    prm = ksa.Params(w.log2n, w.L, w.dnum, w.K, max_batch=K8, device=0)
    primes = prm.primes
    q = primes[: w.L]
    basis = prm.basis(w.L)
    beta, alpha = prm.beta(w.L), prm.alpha(w.L)

    # resident inputs: rotating ciphertext / output buffers, one key
    ct_bytes = K8 * 2 * w.L * w.N * 4
    nbuf = max(2, int(np.ceil(args.buffers_gib * (1 << 30) / (2 * ct_bytes))))
    nbuf += -nbuf % args.streams  # a multiple of the streams: a buffer is reused only by the stream that used it last
    base = ki.ciphertexts(w.index, q, w.N, K8)
    cts, outs = [], []
    for i in range(nbuf):
        t = ksa.to_device(base, 0)
        if i:
            t = torch.roll(t, shifts=i, dims=-1).contiguous()  # distinct contents, same distribution
        cts.append(t)
        outs.append(torch.empty((1, K8, 2, w.L, w.N), dtype=torch.int32, device="cuda:0"))
    evk_b = ksa.to_device(ki.uniform_key_b(w.index, 0, beta, basis, w.N), 0)
    evk_a = ksa.to_device(ki.uniform_key_b(w.index, 1, beta, basis, w.N), 0)  # stands in for a stored a half
    seed = ki.key_seed(w.index, 0)
    torch.cuda.synchronize()

    # independent batches in flight on several streams (default priority), each call
    # with its own workspace (the arena serves one stream at a time); three measured
    # fastest: a fourth shares the process's four hardware queues with the null stream
    S = args.streams
    streams = [torch.cuda.Stream() for _ in range(S)]
    ws_bytes = prm.workspace_bytes(w.L)
    workspaces = [torch.empty((ws_bytes + 3) // 4, dtype=torch.int32, device="cuda:0") for _ in range(S)]

    def step(i, batch, stored=False, ws=None):
        ct = cts[i % nbuf][:batch]
        out = outs[i % nbuf][:, :batch]
        if stored:
            ksa.keyswitch_ex(prm, ct, [evk_b], [1], w.L, evk_a=[evk_a], out=out, workspace=ws)
        else:
            ksa.keyswitch_ex(prm, ct, [evk_b], [1], w.L, seeds=[seed], out=out, workspace=ws)

    def timed_streams(batch, stored=False, steps=args.steps):
        """Steps dealt round-robin to the streams; the region opens with an event that
        every stream waits for and closes when all of them are done."""
        def issue(i):
            with torch.cuda.stream(streams[i % S]):
                step(i, batch, stored, workspaces[i % S])

        for i in range(args.warmup):
            issue(i)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(streams[0])
        for st in streams[1:]:
            st.wait_event(start)
        for i in range(steps):
            issue(i)
        for st in streams[1:]:
            joined = torch.cuda.Event()
            joined.record(st)
            streams[0].wait_event(joined)
        end.record(streams[0])
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    per_step = {}

    def timed(batch, stored=False, steps=args.steps, record=True):
        for i in range(args.warmup):
            step(i, batch, stored)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        t0 = time.perf_counter()
        ev[0].record()
        for i in range(steps):
            step(i, batch, stored)
            ev[i + 1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = ev[0].elapsed_time(ev[-1])
        d = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
        # the first timed region of each variant (the later one runs under the library's profiling)
        if record:
            per_step.setdefault((batch, stored), {"min": round(d[0], 4), "median": round(d[len(d) // 2], 4),
                                                  "max": round(d[-1], 4)})
        return ms / steps, wall

    def spin_up():
        """Untimed batch-8 steps: the engine clock ramps up over the first milliseconds
        of sustained load, and every timed leg should see the loaded GPU."""
        for i in range(int(args.spinup_ms / 0.5)):
            step(i, K8)
        torch.cuda.synchronize()

    spin_up()
    ms8, wall8 = timed(K8)
    ms1, _ = timed(1)
    ms8s, _ = timed(K8, stored=True)
    ms1s, _ = timed(1, stored=True)
    print(f"[bench] one stream: k=8 {ms8:.3f} ms/step, k=1 {ms1:.3f}, stored k=8 {ms8s:.3f}, stored k=1 {ms1s:.3f}",
          file=sys.stderr, flush=True)
    if S > 1:
        spin_up()
        ms8_2, ms1_2 = timed_streams(K8), timed_streams(1)
        ms8s_2, ms1s_2 = timed_streams(K8, stored=True), timed_streams(1, stored=True)
        print(f"[bench] {S} streams: k=8 {ms8_2:.3f} ms/step, k=1 {ms1_2:.3f}, stored k=8 {ms8s_2:.3f}, "
              f"stored k=1 {ms1s_2:.3f}", file=sys.stderr, flush=True)
    else:
        ms8_2, ms1_2, ms8s_2, ms1s_2 = ms8, ms1, ms8s, ms1s
    head = ms8  # the headline: batch-8 key switches, one after another on one stream

    # steady state: many consecutive batch-8 steps on one stream (the clock settles
    # under sustained load)
    long_ms = None
    if args.long_steps > 0:
        long_ms, _ = timed(K8, steps=args.long_steps, record=False)
        print(f"[bench] steady state: k=8 {long_ms:.3f} ms/step over {args.long_steps} steps", file=sys.stderr,
              flush=True)

    # per-kernel HIP-event timings over a timed region of the same k=8 steps
    ksa.profile_begin(prm)
    ms8p, _ = timed(K8)
    kstats = ksa.profile_end(prm)
    kernels = {k: {"launches": n, "avg_us": 1000.0 * t / n, "share": t / (ms8p * args.steps)}
               for k, (n, t) in sorted(kstats.items(), key=lambda kv: -kv[1][1])}
    ksa.profile_begin(prm)
    timed(K8, stored=True)
    kstats_stored = ksa.profile_end(prm)
    ksa.profile_begin(prm)
    ms1p, _ = timed(1)
    kstats_k1 = ksa.profile_end(prm)

    def timed_calls(fn, steps):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def profiled(fn, families):
        ksa.profile_begin(prm)
        try:
            for i in range(10):
                fn(i)
        finally:
            st = ksa.profile_end(prm)
        return {k: round(1000.0 * t / n, 3) for k, (n, t) in st.items() if k in families}

    def keygen_leg():
        # key generation of the same relinearisation key on the GPU (pc_keygen): synthetic
        # secret / error residues of the right shape (timing does not depend on their values)
        s_coef = ksa.to_device(ki.uniform_key_b(w.index, 2, 1, basis, w.N)[0], 0)
        e_coef = ksa.to_device(ki.uniform_key_b(w.index, 3, beta, basis, w.N), 0)
        kg_out = torch.empty((beta, w.L + w.K, w.N), dtype=torch.int32, device="cuda:0")
        ms = timed_calls(lambda i: ksa.keygen(prm, seed, w.L, 1, s_coef, e_coef, out=kg_out), 10)
        return {"keys_per_s": round(1000.0 / ms, 1), "ms_per_key": round(ms, 4)}

    def hmult_leg():
        # homomorphic multiplication of 8 ciphertext pairs at the top level around the same
        # key switch (pc_hmult: tensor, relinearise d2, rescale); per-kernel times profiled
        hm_out = torch.empty((K8, 2, w.L - 1, w.N), dtype=torch.int32, device="cuda:0")

        def hm_step(i):
            ksa.hmult(prm, cts[i % nbuf], cts[(i + 1) % nbuf], evk_b, seed, w.L, out=hm_out)

        ms = timed_calls(hm_step, args.steps)
        fams = ("tensor", "rescale_gather", "rescale_col", "moddown_fwd_blk", "moddown_rescale")
        return {"hmults_per_s": round(K8 * 1000.0 / ms, 1), "ms_per_call": round(ms, 4),
                "kernel_avg_us": profiled(hm_step, fams)}

    def bsgs_leg():
        # double-hoisted BSGS linear transform of one ciphertext, 4 x 4 diagonals
        # (baby X^(5^i), i=1..3; giant X^(5^(4j)), j=1..3), uniform diagonals and key b halves
        wb = ki.WORKLOADS["bsgs16"]
        n1, n2 = wb.extra["n1"], wb.extra["n2"]
        lt_keys = [ksa.to_device(ki.uniform_key_b(wb.index, k, beta, basis, w.N), 0) for k in range(len(wb.galois))]
        lt_seeds = [ki.key_seed(wb.index, k) for k in range(len(wb.galois))]
        lt_diag = ksa.to_device(ki.uniform_diagonals(wb.index, n2, n1, basis, w.N), 0)
        lt_out = torch.empty((2, w.L, w.N), dtype=torch.int32, device="cuda:0")

        def lt_step(i):
            ksa.linear_transform(prm, cts[i % nbuf][0], lt_diag, w.L,
                                 baby_b=lt_keys[: n1 - 1], baby_seeds=lt_seeds[: n1 - 1],
                                 baby_galois=wb.galois[: n1 - 1], giant_b=lt_keys[n1 - 1:],
                                 giant_seeds=lt_seeds[n1 - 1:], giant_galois=wb.galois[n1 - 1:], out=lt_out)

        ms = timed_calls(lt_step, args.steps)
        return {"transforms_per_s": round(1000.0 / ms, 1), "ms_per_call": round(ms, 4),
                "key_switches": (n1 - 1) + (n2 - 1), "kernel_avg_us": profiled(lt_step, ("bsgs_baby", "bsgs_giant"))}

    def leg(fn):
        """An auxiliary measurement; a failure is reported in the line instead of losing it."""
        try:
            return fn()
        except Exception as exc:  # noqa: BLE001 - reported, not hidden
            print(f"[bench] {fn.__name__} failed: {exc!r}", file=sys.stderr, flush=True)
            return {"error": repr(exc)}

    keygen_res = leg(keygen_leg)
    hmult_res = leg(hmult_leg)
    bsgs_res = leg(bsgs_leg)
    # measured stream-copy bandwidth (context for the 8 TB/s peak): 1 GiB read + 1 GiB write;
    # left out of counter runs, whose byte calibration needs the 256 MiB copy to be the only one
    copy_gbs = None
    if not args.calibrate_copy:
        csrc = torch.ones(1 << 28, dtype=torch.int32, device="cuda:0")
        cdst = torch.empty_like(csrc)
        for _ in range(3):
            cdst.copy_(csrc)
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(10):
            cdst.copy_(csrc)
        c1.record()
        torch.cuda.synchronize()
        copy_gbs = round(2.0 * csrc.numel() * 4 / (c0.elapsed_time(c1) / 10 * 1e-3) / 1e9, 1)
        del csrc, cdst
    prm.close()
    del cts, outs, workspaces
    torch.cuda.empty_cache()
    others = None if args.no_configs else leg(lambda: other_configs(ksa, torch, args))
    kernels_stored = {k: round(1000.0 * t / n, 3) for k, (n, t) in sorted(kstats_stored.items(), key=lambda kv: -kv[1][1])}
    kernels_k1 = {k: round(1000.0 * t / n, 3) for k, (n, t) in sorted(kstats_k1.items(), key=lambda kv: -kv[1][1])}
    dom = next(iter(kernels))
    roofs = {k: kernel_roofline(k, v["avg_us"], w, K8, beta, alpha) for k, v in kernels.items()}
    from key_switching_amd import profiling
    traffic_md = os.path.join(ROOT, "profiles", "keyswitch_n16_k8_traffic.md")
    valu_md = os.path.join(ROOT, "profiles", "keyswitch_n16_k8_valu.md")
    rd = roofs[dom]
    if rd["alu_frac"] >= rd["hbm_frac"]:
        roofline = {"bound": "alu", "achieved": rd["alu_tops"], "peak": round(INT32_PEAK_TOPS, 2), "unit": "TOP/s",
                    "frac": rd["alu_frac"]}
    else:
        roofline = {"bound": "hbm", "achieved": rd["hbm_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": rd["hbm_frac"]}
    traffic = profiling.read_traffic(traffic_md, dom)
    step_s = head * 1e-3
    path_bytes = sum(r["alg_bytes"] for r in roofs.values())
    path_ops = sum(r["alg_ops"] for r in roofs.values())
    path = {"alg_bytes_per_step": path_bytes, "alg_ops_per_step": path_ops,
            "hbm_frac": round(path_bytes / step_s / 1e9 / HBM_PEAK_GBS, 4),
            "alu_frac": round(path_ops / step_s / 1e12 / INT32_PEAK_TOPS, 4),
            "alu_frac_streams": round(path_ops / (ms8_2 * 1e-3) / 1e12 / INT32_PEAK_TOPS, 4),
            "alu_frac_steady_state": (round(path_ops / (long_ms * 1e-3) / 1e12 / INT32_PEAK_TOPS, 4)
                                      if long_ms else None),
            "k1_alu_frac_one_stream": path_fractions([(w.N, w.L, w.K, alpha, beta, 1, 1, True)], ms1)["alu_frac"]}
    roofline.update({"traffic": None if traffic is None else round(traffic), "kernel": dom,
                     "alg_bytes_per_launch": rd["alg_bytes"], "alg_ops_per_launch": rd["alg_ops"],
                     "hbm_frac": rd["hbm_frac"], "alu_frac": rd["alu_frac"], "avg_us": rd["avg_us"],
                     "valu_issued_over_alg": profiling.read_valu_ratio(valu_md, dom),
                     "path_alu_frac": path["alu_frac"]})

    result = {
        "metric": METRIC,
        "value": round(K8 * 1000.0 / head, 1),
        "unit": "key switches/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": "n16: N=2^16, L=24 q-primes (31-bit), dnum=4 (alpha=6), K=6, relinearisation key, "
                               "a half regenerated in-kernel (ChaCha12), batch k=8, one stream",
                   "N": w.N, "L": w.L, "dnum": w.dnum, "K": w.K, "batch": K8, "buffers": nbuf},
        "k1_ks_per_s": round(1000.0 / ms1, 1),
        "k1_note": "batch 1, one call at a time on one stream (each call's kernels wait for the previous call)",
        "variants": {
            "streams": args.streams,
            "k8_chacha_independent_calls_on_streams": {
                "ks_per_s": round(K8 * 1000.0 / ms8_2, 1), "ms_per_call": round(ms8_2, 4),
                "note": f"independent batch-8 calls dealt to {args.streams} streams"},
            "k8_stored_independent_calls_on_streams": {"ks_per_s": round(K8 * 1000.0 / ms8s_2, 1),
                                                       "ms_per_call": round(ms8s_2, 4)},
            "k1_chacha_independent_calls_on_streams": {
                "ks_per_s": round(1000.0 / ms1_2, 1), "ms_per_call": round(ms1_2, 4),
                "note": f"independent batch-1 calls dealt to {args.streams} streams (up to {args.streams} in flight)"},
            "k1_stored_independent_calls_on_streams": {"ks_per_s": round(1000.0 / ms1s_2, 1),
                                                       "ms_per_call": round(ms1s_2, 4)},
            "k8_chacha_one_stream": {"ks_per_s": round(K8 * 1000.0 / ms8, 1), "ms_per_call": round(ms8, 4)},
            "k1_chacha_one_stream": {"ks_per_s": round(1000.0 / ms1, 1), "ms_per_call": round(ms1, 4)},
            "k8_stored_one_stream": {"ks_per_s": round(K8 * 1000.0 / ms8s, 1), "ms_per_call": round(ms8s, 4)},
            "k1_stored_one_stream": {"ks_per_s": round(1000.0 / ms1s, 1), "ms_per_call": round(ms1s, 4)},
            "k8_chacha_steady_state": ({"ks_per_s": round(K8 * 1000.0 / long_ms, 1), "ms_per_call": round(long_ms, 4),
                                        "steps": args.long_steps} if long_ms else None),
            "k8_chacha_profiled": {"ms_per_call": round(ms8p, 4)},
            "k1_chacha_profiled": {"ms_per_call": round(ms1p, 4)},
            "keygen_relin_key": keygen_res,
            "hmult_k8": hmult_res,
            "bsgs_4x4": bsgs_res,
        },
        "ms_per_step_k8_one_stream": per_step[(K8, False)],
        "ms_per_step_k1_one_stream": per_step[(1, False)],
        "copy_gbs_measured": copy_gbs,
        "other_configs": others,
        "kernels": {k: {**{kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()},
                        "hbm_frac": roofs[k]["hbm_frac"], "alu_frac": roofs[k]["alu_frac"]}
                    for k, v in kernels.items()},
        "path_roofline": path,
        "kernels_k8_stored_avg_us": kernels_stored,
        "kernels_k1_avg_us": kernels_k1,
        "roofline": roofline,
        "wall_s_k8": round(wall8, 3),
    }
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


def _time_calls(torch, fn, steps, warmup=3):
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def other_configs(ksa, torch, args, steps=10, only=None):
    """Key switches per second on the other workloads (uniform b halves standing in for
    real ones; the a halves regenerated in-kernel, or read from a stored copy).

    hoist16: one N=2^16 ciphertext, ModUp once, 16 rotation keys (also drawn from a
    packed and a full key bundle); levels16: 8 ciphertexts switched independently by the
    X^5 and X^-1 keys at each level; n17: 8 N=2^17, L=40 ciphertexts, relinearised then
    rotated by X^5. ``only`` limits the run to one of them (profiler runs).
    """
    out = {}
    if only in (None, "hoist16"):
        w = ki.WORKLOADS["hoist16"]
        R = len(w.galois)
        with ksa.Params(w.log2n, w.L, w.dnum, w.K, max_batch=1, max_hoist=R, device=0) as prm:
            basis, beta = prm.basis(w.L), prm.beta(w.L)
            keys = [ksa.to_device(ki.uniform_key_b(w.index, k, beta, basis, w.N), 0) for k in range(R)]
            akeys = [ksa.to_device(ki.uniform_key_b(w.index, 100 + k, beta, basis, w.N), 0) for k in range(R)]
            seeds = [ki.key_seed(w.index, k) for k in range(R)]
            ct = ksa.to_device(ki.ciphertexts(w.index, prm.primes[: w.L], w.N, 1), 0)
            res = torch.empty((R, 1, 2, w.L, w.N), dtype=torch.int32, device="cuda:0")
            one = (w.N, w.L, w.K, prm.alpha(w.L), beta, 1, R, True)
            ms = _time_calls(torch, lambda i: ksa.keyswitch_ex(prm, ct, keys, w.galois, w.L, seeds=seeds, out=res),
                             steps)
            mss = _time_calls(torch, lambda i: ksa.keyswitch_ex(prm, ct, keys, w.galois, w.L, evk_a=akeys, out=res),
                              steps)
            d = {"ks_per_s": round(R * 1000.0 / ms, 1), "ms_per_call": round(ms, 4), "key_switches_per_call": R,
                 "path": path_fractions([one], ms),
                 "stored": {"ks_per_s": round(R * 1000.0 / mss, 1), "ms_per_call": round(mss, 4),
                            "path": path_fractions([one], mss, stored=True)}}
            # the same keys from key bundles: packed (b halves + seeds) and full (a halves stored too)
            for name, full in (("bundle_packed", False), ("bundle_full", True)):
                with ksa.KeySet(prm, w.L, w.galois, full=full) as bundle:
                    for k in range(R):
                        bundle.set(k, keys[k], seeds[k])
                    idx = list(range(R))
                    msb = _time_calls(torch, lambda i: ksa.keyswitch_keyset(prm, bundle, ct, idx, w.L, out=res),
                                      steps)
                    d[name] = {"ks_per_s": round(R * 1000.0 / msb, 1), "ms_per_call": round(msb, 4),
                               "device_bytes": bundle.device_bytes(), "key_half_bytes": bundle.key_bytes()}
            out["hoist16"] = d
            del keys, akeys, ct, res
    if only in (None, "levels16"):
        w = ki.WORKLOADS["levels16"]
        with ksa.Params(w.log2n, w.L, w.dnum, w.K, max_batch=8, device=0) as prm:
            base = ki.ciphertexts(w.index, prm.primes[: w.L], w.N, 8)
            per_level, per_level_path = {}, {}
            for level in w.levels:
                basis, beta = prm.basis(level), prm.beta(level)
                keys = [ksa.to_device(ki.uniform_key_b(w.index, 10 * level + k, beta, basis, w.N), 0)
                        for k in range(2)]
                seeds = [ki.key_seed(w.index, 10 * level + k) for k in range(2)]
                ct = ksa.to_device(np.ascontiguousarray(base[:, :, :level]), 0)
                res = torch.empty((1, 8, 2, level, w.N), dtype=torch.int32, device="cuda:0")

                def one_level(i):
                    for k in range(2):  # each key on its own: 16 single key switches
                        ksa.keyswitch_ex(prm, ct, [keys[k]], [w.galois[k]], level, seeds=[seeds[k]], out=res)

                ms = _time_calls(torch, one_level, steps)
                per_level[str(level)] = round(16 * 1000.0 / ms, 1)
                one = (w.N, level, w.K, prm.alpha(level), beta, 8, 1, True)
                per_level_path[str(level)] = path_fractions([one, one], ms)
                del keys, ct, res
            out["levels16"] = {"ks_per_s_by_level": per_level, "path_by_level": per_level_path}
    if only in (None, "n17"):
        w = ki.WORKLOADS["n17"]
        with ksa.Params(w.log2n, w.L, w.dnum, w.K, max_batch=8, device=0) as prm:
            basis, beta = prm.basis(w.L), prm.beta(w.L)
            keys = [ksa.to_device(ki.uniform_key_b(w.index, k, beta, basis, w.N), 0) for k in range(2)]
            akeys = [ksa.to_device(ki.uniform_key_b(w.index, 100 + k, beta, basis, w.N), 0) for k in range(2)]
            seeds = [ki.key_seed(w.index, k) for k in range(2)]
            ct = ksa.to_device(ki.ciphertexts(w.index, prm.primes[: w.L], w.N, 8), 0)
            mid = torch.empty((1, 8, 2, w.L, w.N), dtype=torch.int32, device="cuda:0")
            res = torch.empty_like(mid)

            def chain(i, stored=False):
                kw0 = {"evk_a": [akeys[0]]} if stored else {"seeds": [seeds[0]]}
                kw1 = {"evk_a": [akeys[1]]} if stored else {"seeds": [seeds[1]]}
                ksa.keyswitch_ex(prm, ct, [keys[0]], [w.galois[0]], w.L, out=mid, **kw0)
                ksa.keyswitch_ex(prm, mid[0], [keys[1]], [w.galois[1]], w.L, out=res, **kw1)

            ms = _time_calls(torch, chain, steps)
            mss = _time_calls(torch, lambda i: chain(i, stored=True), steps)
            ksa.profile_begin(prm)
            try:
                for i in range(3):
                    chain(i)
            finally:
                kst = ksa.profile_end(prm)
            chain_kernels = {k: round(1000.0 * t / n, 2) for k, (n, t) in sorted(kst.items(), key=lambda kv: -kv[1][1])}
            one = (w.N, w.L, w.K, prm.alpha(w.L), beta, 8, 1, True)
            traffic = None
            try:
                from key_switching_amd import profiling
                traffic = profiling.read_ip_traffic(os.path.join(ROOT, "profiles", "keyswitch_n17_chain_traffic.md"))
            except Exception:  # noqa: BLE001 - the summary is optional context
                traffic = None
            out["n17"] = {"ks_per_s": round(16 * 1000.0 / ms, 1), "ms_per_call": round(ms, 4),
                          "key_switches_per_call": 16, "path": path_fractions([one, one], ms),
                          "stored": {"ks_per_s": round(16 * 1000.0 / mss, 1), "ms_per_call": round(mss, 4),
                                     "path": path_fractions([one, one], mss, stored=True)},
                          "key_half_bytes": beta * (w.L + w.K) * w.N * 4,
                          "kernel_avg_us": chain_kernels,
                          "inner_product_traffic_bytes": traffic}
            del keys, akeys, ct, mid, res
    return out


if __name__ == "__main__":
    main()
