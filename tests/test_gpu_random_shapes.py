"""Seeded random batch shapes, every row against the float64 oracle.

Each case draws, from its own PCG64 seed, a batch of 1-5 requests with
random query and prefix lengths (empty queries, single tokens, lengths off
the page, tile and partition sizes), a head layout, a head dim and a split
size, and runs the paged prefill (or decode) through the C ABI. A second
run of the same batch on re-permuted page ids must give the same bits.
"""
import numpy as np
import pytest

import workloads as W
from gpu_util import assert_parity, bits_equal, run_decode, run_prefill, say

pytestmark = pytest.mark.gpu
DEV = "cuda"

HEADS = [
    dict(num_qo_heads=32, num_kv_heads=8, head_dim=128),
    dict(num_qo_heads=8, num_kv_heads=8, head_dim=128),
    dict(num_qo_heads=16, num_kv_heads=2, head_dim=128),
    dict(num_qo_heads=16, num_kv_heads=8, head_dim=64),
    dict(num_qo_heads=4, num_kv_heads=1, head_dim=64),
]
SPLITS = [64, 192, 1024, 4096]


def random_prefill_case(seed: int):
    g = np.random.Generator(np.random.PCG64(1000 + seed))
    heads = HEADS[int(g.integers(len(HEADS)))]
    split = SPLITS[int(g.integers(len(SPLITS)))]
    reqs = []
    for r in range(int(g.integers(1, 6))):
        qo = int(g.choice([0, 1, int(g.integers(2, 64)), int(g.integers(64, 330))]))
        prefix = int(g.choice([0, int(g.integers(1, 300)), int(g.integers(300, 1300))]))
        reqs.append(W.Request(qo, max(qo + prefix, 1), 5000 + 97 * seed + r))
    if all(r.qo_len == 0 for r in reqs):
        reqs[0] = W.Request(1, reqs[0].kv_len, reqs[0].seed)
    return reqs, heads, split


@pytest.mark.parametrize("seed", range(16))
def test_random_prefill(seed):
    reqs, heads, split = random_prefill_case(seed)
    shape = [(r.qo_len, r.kv_len) for r in reqs]
    say(f"random prefill seed {seed}: {shape} {heads} split {split}")
    b = W.make_batch(reqs, num_pages=1024, batch_seed=70 + seed, device=DEV, **heads)
    out, lse = run_prefill(b, split=split)
    assert_parity(out, lse, b, what=f"random prefill seed {seed}")
    # same requests on other pages: the same bits
    b2 = W.make_batch(reqs, num_pages=1024, batch_seed=170 + seed, device=DEV, **heads)
    out2, lse2 = run_prefill(b2, split=split)
    assert bits_equal(out, out2) and bits_equal(lse, lse2), "page relocation changed bits"


@pytest.mark.parametrize("seed", range(8))
def test_random_decode(seed):
    g = np.random.Generator(np.random.PCG64(2000 + seed))
    heads = HEADS[int(g.integers(len(HEADS)))]
    ctx = [int(g.integers(1, 9000)) for _ in range(int(g.integers(1, 12)))]
    say(f"random decode seed {seed}: ctx {ctx} {heads}")
    b = W.decode_batch(len(ctx), ctx_lens=ctx, num_pages=8192, device=DEV, head=heads)
    out, lse = run_decode(b)
    assert_parity(out, lse, b, what=f"random decode seed {seed}")
