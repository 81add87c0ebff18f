"""The cases where a q-tile choice made from batch statistics breaks chunk
invariance (sglang PR #43612, Summary: a tiny last chunk, a chunk batched
with many 1-token extends, an off-grid prefix-cache hit landing on a
different tile). Here the tile shape is fixed and each row's arithmetic does
not depend on the tile holding it, so every case must reproduce the
unchunked rows bit for bit, and meet oracle parity. The prefix lengths 1,
511, 2048 and 4097 are the ones the deterministic-inference prefix test uses
(sglang PR #10417, Reproduction)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import assert_parity, bits_equal, run_prefill, sample_rows, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def seq():
    """One 6000-token request (Qwen3-8B heads) and its unchunked prefill."""
    s = W.make_sequence(6000, seed=17, num_pages=1024, device=DEV)
    out, lse = run_prefill(s.batch)
    return s, out, lse


def test_unchunked_reference_parity(seq):
    """The unchunked 6000-token rows every case below is compared with meet
    oracle parity on the first and last 128 rows, every 61st row, and the
    rows around each chunk and prefix boundary the cases use."""
    s, of, lf = seq
    say("6000-token unchunked reference vs oracle (sampled rows)")
    rows = set(sample_rows(6000).tolist())
    for c in (1, 511, 2048, 2560, 3200, 4097, 5888, 5997):
        rows |= {max(0, c - 1), c, min(5999, c + 1)}
    assert_parity(of, lf, s.batch, [0], {0: np.array(sorted(rows))},
                  what="6000-token unchunked")


def test_tiny_last_chunk(seq):
    s, of, lf = seq
    say("tiny last chunk: 256-token chunks up to 5888, then 112, then 3 + ... ")
    bounds = W.chunk_bounds(5888, 256) + [(5888, 5997), (5997, 6000)]
    outs, lses = [], []
    for lo, hi in bounds:
        o, l = run_prefill(s.chunk(lo, hi))
        outs.append(o)
        lses.append(l)
    assert bits_equal(torch.cat(outs), of) and bits_equal(torch.cat(lses), lf)


def test_chunk_batched_with_many_one_token_extends(seq):
    """A 640-token chunk (positions 2560..3199) shares the batch with 48
    single-token extends of other requests; its rows equal the unchunked
    rows."""
    s, of, lf = seq
    say("chunk batched with 48 one-token extends")
    lo, hi = 2560, 3200
    ch = s.chunk(lo, hi)
    rng = np.random.Generator(np.random.PCG64(23))
    extends = [W.Request(1, int(c), 900 + i) for i, c in
               enumerate(rng.integers(1, 9000, size=48))]
    # the chunk goes in the middle of the batch, with its own pages placed
    # into a pool shared with the extends
    k_seq = s.batch.k_pool.view(-1, 8, 128)
    v_seq = s.batch.v_pool.view(-1, 8, 128)
    pages = s.batch.page_table[: (hi + 15) // 16].astype(np.int64)
    slots = (pages[:, None] * 16 + np.arange(16)[None, :]).reshape(-1)[:hi]
    idx = torch.as_tensor(slots, device=DEV)
    q_list, k_list, v_list, qo, kv = [], [], [], [], []
    for r in extends[:24]:
        k, v, q = W.draw_request(r, 32, 8, 128, DEV)
        q_list.append(q), k_list.append(k), v_list.append(v), qo.append(1), kv.append(r.kv_len)
    q_list.append(ch.q), k_list.append(k_seq[idx]), v_list.append(v_seq[idx])
    qo.append(hi - lo), kv.append(hi)
    for r in extends[24:]:
        k, v, q = W.draw_request(r, 32, 8, 128, DEV)
        q_list.append(q), k_list.append(k), v_list.append(v), qo.append(1), kv.append(r.kv_len)
    b = W.assemble_batch(qo, kv, q_list, k_list, v_list, num_pages=65536, batch_seed=29,
                         device=DEV)
    out, lse = run_prefill(b)
    r0 = int(b.qo_indptr[24])
    assert bits_equal(out[r0: r0 + hi - lo], of[lo:hi])
    assert bits_equal(lse[r0: r0 + hi - lo], lf[lo:hi])
    assert_parity(out, lse, b, [0, 24, 48], what="chunk among 1-token extends")


@pytest.mark.parametrize("prefix", [1, 511, 2048, 4097])
def test_prefix_cache_hit(seq, prefix):
    """Prefix of `prefix` tokens already cached (off the 128 grid for 1, 511
    and 4097); the remaining 6000 - prefix tokens in one call equal the
    unchunked rows."""
    s, of, lf = seq
    say(f"prefix-cache hit at {prefix}")
    o, l = run_prefill(s.chunk(prefix, 6000))
    assert bits_equal(o, of[prefix:]) and bits_equal(l, lf[prefix:])
    if prefix in (1, 4097):
        rows = {0: np.array([0, 1, 2, 63, 64, 1000, 6000 - prefix - 1])}
        assert_parity(o, l, s.chunk(prefix, 6000), [0], rows, what=f"prefix {prefix}")
