"""Seeded random shapes through the whole decode and prefill paths, against the CPU oracle.

Each case draws its own request count, ragged context lengths (block multiples and partial tails),
queries per request, KV heads, group size, head and index dims and k from a seeded generator, so
the fixed cases elsewhere are complemented by combinations nobody picked by hand.  The bars are
the same as in test_gpu_decode.py and test_gpu_prefill.py.
"""
import numpy as np
import pytest

import msa_inputs as mi
from _gpu import announce, setup
from test_gpu_decode import _check_against_oracle as check_decode
from test_gpu_prefill import _check_against_oracle as check_prefill

pytestmark = pytest.mark.gpu


def _ctx(rng, lo, hi):
    L = int(rng.integers(lo, hi + 1))
    return L - L % 128 if rng.random() < 0.25 and L >= 128 else L   # some exact block multiples


def _common(rng, kv_heads=(1, 2, 4)):
    Hkv = int(rng.choice(kv_heads))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    while Hkv * G > 128:
        G //= 2
    return dict(Hq=Hkv * G, Hkv=Hkv, D=int(rng.choice([64, 128])), Di=int(rng.choice([64, 128])),
                k=int(rng.integers(1, 65)))


def decode_case(seed):
    """Up to 8 requests of up to 16 queries; KV heads up to 16 (Hkv*Di > 1024 takes the direct
    scorer); planted hot blocks in some cases."""
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.integers(1, 9))
    ctx = [_ctx(rng, 1, 8000) for _ in range(B)]
    nq = [int(rng.integers(1, min(16, L) + 1)) for L in ctx]
    hot = int(rng.choice([0, 0, 4]))
    return mi.small_workload(ctx, nq, seed=5000 + seed, hot_per_group=hot,
                             **_common(rng, kv_heads=(1, 2, 3, 4, 8, 16)))


def prefill_case(seed):
    rng = np.random.default_rng(6000 + seed)
    B = int(rng.integers(1, 4))
    ctx = [_ctx(rng, 40, 2500) for _ in range(B)]
    nq = [int(rng.integers(17, min(200, L) + 1)) if L > 17 else L for L in ctx]
    return mi.small_workload(ctx, nq, seed=6000 + seed, **_common(rng))


@pytest.mark.parametrize("seed", range(10))
def test_random_decode_shapes(seed):
    wl = decode_case(seed)
    announce("random decode", f"seed {seed}: ctx {wl.ctx_lens} nq {wl.q_counts} Hkv {wl.Hkv} G {wl.G} "
                              f"D {wl.D} Di {wl.Di} k {wl.k}")
    dev, cpu = setup(wl)
    check_decode(dev, cpu)


@pytest.mark.parametrize("seed", range(10))
def test_random_prefill_shapes(seed):
    wl = prefill_case(seed)
    announce("random prefill", f"seed {seed}: ctx {wl.ctx_lens} nq {wl.q_counts} Hkv {wl.Hkv} G {wl.G} "
                               f"D {wl.D} Di {wl.Di} k {wl.k}")
    dev, cpu = setup(wl)
    check_prefill(dev, cpu)
