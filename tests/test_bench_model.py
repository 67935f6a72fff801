"""The benchmark's roofline model and command-line contract (CPU only).

The algorithmic byte and operation counts are closed forms of the workload's
shape; these checks pin them by hand-computed totals so that a change to the
model cannot silently move the reported roofline fractions.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import ks_inputs as ki  # noqa: E402

LIMB16 = 4 << 16  # bytes of one N = 2^16 limb


def test_headline_totals():
    """N=2^16, L=24, dnum=4 (alpha 6, 4 digits), K=6, batch 8: per step."""
    w = ki.WORKLOADS["n16"]
    nbytes = sum(bench.alg_bytes_per_launch(k, w, 8, 4, 6) for k in bench.KERNELS)
    nops = sum(bench.alg_ops_per_launch(k, w, 8, 4, 6) for k in bench.KERNELS)
    # limbs: ModUp 8*(48 + 48 + 24+96 + 192) = 3264; IP 8*(96+24) + 4*30 + 8*60 = 1560;
    # ModDown 8*2*(12 + 12 + 30 + 72) + 8*24 = 2208 -> 7032 limbs
    assert nbytes == 7032 * LIMB16
    # inner product: 2 sums of dot_ops(4) = 10 per position and item, 8 items x 30 limbs
    assert bench.alg_ops_per_launch("inner_product", w, 8, 4, 6) == (
        8 * 30 * (1 << 16) * 2 * 10 + 30 * (1 << 16) * 4 * (bench.OPS_REDC + bench.OPS_CHACHA12_BLOCK / 8
                                                           + bench.OPS_WORDPAIR))
    assert nops == 10739515392


def test_model_scales_with_batch_and_keys():
    N, L, K = 1 << 16, 24, 6
    one = {k: bench.alg_bytes(k, N, L, K, 6, 4, 1, 1) for k in bench.KERNELS}
    eight = {k: bench.alg_bytes(k, N, L, K, 6, 4, 8, 1) for k in bench.KERNELS}
    for k in bench.KERNELS:
        if k == "inner_product":  # the key's b half is read once per batch
            assert eight[k] == 8 * one[k] - 7 * 4 * (L + K) * LIMB16
        else:
            assert eight[k] == 8 * one[k]
    # hoisting: ModUp once, the per-key work scales with the keys
    hoist = bench.path_fractions([(N, L, K, 6, 4, 1, 16, True)], 1.0)
    single = bench.path_fractions([(N, L, K, 6, 4, 1, 1, True)], 1.0)
    modup = sum(bench.alg_ops(k, N, L, K, 6, 4, 1, 1) for k in bench.KERNELS if k.startswith("modup"))
    assert hoist["alg_ops_per_call"] == modup + 16 * (single["alg_ops_per_call"] - modup)


def test_n17_passes_split_stages():
    """N=2^17 has an 8-stage column pass and a 9-stage block pass."""
    N = 1 << 17
    col = bench.alg_ops("modup_inv_col", N, 40, 8, 8, 5, 1) - 40 * N * bench.OPS_SHOUP
    blk = bench.alg_ops("modup_inv_blk", N, 40, 8, 8, 5, 1)
    assert col * 9 == blk * 8


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("alpha,dots", [(1, 5), (2, 6), (3, 9), (4, 10), (5, 13), (6, 14)])
def test_dot_product_op_counts(alpha, dots):
    """alpha multiply-adds, a fold after the 4th product and every further pair, one REDC."""
    assert bench.dot_ops(alpha) == dots
