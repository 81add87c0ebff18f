"""Bitwise invariance of the GPU path against itself: batch composition,
decode batch size 1-64, on-grid chunkings, page relocation and run-to-run
repeat. Off-grid chunkings (100-token chunks) must meet oracle parity; their
bit equality with the unchunked call is recorded, not required."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import (assert_parity, bits_equal, run_decode, run_prefill,
                      sample_rows, say)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def rows_of(b, r):
    return slice(int(b.qo_indptr[r]), int(b.qo_indptr[r + 1]))


def test_prefill_batch_composition():
    """A request's bits are the same alone and in two different batches (other
    neighbours, other position, other page ids)."""
    say("prefill batch composition")
    x = W.Request(700, 1500, 501)
    kw = dict(num_pages=4096, device=DEV, **W.QWEN3_8B)
    alone = W.make_batch([x], batch_seed=1, **kw)
    b1 = W.make_batch([W.Request(33, 33, 502), x, W.Request(1, 4000, 503)],
                      batch_seed=2, **kw)
    b2 = W.make_batch([W.Request(2000, 2000, 504), W.Request(0, 10, 505),
                       W.Request(5, 7, 506), x], batch_seed=3, **kw)
    for split in (4096, 512):
        o0, l0 = run_prefill(alone, split=split)
        o1, l1 = run_prefill(b1, split=split)
        o2, l2 = run_prefill(b2, split=split)
        assert bits_equal(o0, o1[rows_of(b1, 1)]) and bits_equal(l0, l1[rows_of(b1, 1)])
        assert bits_equal(o0, o2[rows_of(b2, 3)]) and bits_equal(l0, l2[rows_of(b2, 3)])


def test_prefill_run_to_run_and_relocation():
    say("qwen prefill repeat + page relocation")
    b = W.qwen_prefill(device=DEV, batch=4, length=2048, num_pages=16384)
    o1, l1 = run_prefill(b)
    for _ in range(4):
        o2, l2 = run_prefill(b)
        assert bits_equal(o1, o2) and bits_equal(l1, l2)
    ragged = W.make_batch([W.Request(77, 300, 403), W.Request(129, 129, 404),
                           W.Request(500, 1100, 406), W.Request(64, 64, 407)],
                          num_pages=512, batch_seed=8, device=DEV, **W.QWEN3_8B)
    for split in (4096, 128):
        r1, rl1 = run_prefill(ragged, split=split)
        for _ in range(4):
            r2, rl2 = run_prefill(ragged, split=split)
            assert bits_equal(r1, r2) and bits_equal(rl1, rl2)
    moved = W.make_batch(b.requests, num_pages=16384, batch_seed=99, device=DEV,
                         **W.QWEN3_8B)
    assert not np.array_equal(moved.page_table, b.page_table)
    o3, l3 = run_prefill(moved)
    assert bits_equal(o1, o3) and bits_equal(l1, l3)


def chunked(seq, bounds, split=4096):
    outs, lses = [], []
    for lo, hi in bounds:
        o, l = run_prefill(seq.chunk(lo, hi), split=split)
        outs.append(o)
        lses.append(l)
    return torch.cat(outs), torch.cat(lses)


def test_tiny_chunk_128_plus_172():
    say("tiny chunk invariance 128 + 172")
    seq = W.tiny_sequence(device=DEV)
    of, lf = run_prefill(seq.batch)
    oc, lc = chunked(seq, [(0, 128), (128, 300)])
    assert bits_equal(of, oc) and bits_equal(lf, lc)
    for split in (64, 128):
        of2, lf2 = run_prefill(seq.batch, split=split)
        oc2, lc2 = chunked(seq, [(0, 128), (128, 300)], split=split)
        assert bits_equal(of2, oc2) and bits_equal(lf2, lc2)


def test_tiny_off_grid_chunks_parity():
    say("tiny off-grid chunks (100) parity")
    seq = W.tiny_sequence(device=DEV)
    of, lf = run_prefill(seq.batch)
    oc, lc = chunked(seq, W.chunk_bounds(300, 100))
    full = seq.batch
    assert_parity(oc, lc, full, what="tiny 100-chunks vs oracle")
    say(f"tiny 100-chunks bit-equal to unchunked: {bits_equal(of, oc) and bits_equal(lf, lc)}")


def test_16k_chunk_invariance():
    """One 16384-token request, Qwen head shape: 256-token chunks (on the 128
    grid) reproduce the unchunked call bit for bit; 100-token chunks (off
    grid) meet oracle parity and their bit equality is recorded."""
    say("16k unchunked")
    seq = W.make_sequence(16384, seed=3, num_pages=4096, device=DEV)
    of, lf = run_prefill(seq.batch)
    rows = {0: sample_rows(16384, edge=128, every=61)}
    assert_parity(of, lf, seq.batch, [0], rows, what="16k unchunked (sampled)")
    say("16k in 256-token chunks")
    oc, lc = chunked(seq, W.chunk_bounds(16384, 256))
    assert bits_equal(of, oc), "256-token chunks differ from the unchunked call"
    assert bits_equal(lf, lc)
    say("16k in 100-token chunks")
    o1, l1 = chunked(seq, W.chunk_bounds(16384, 100))
    assert_parity(o1, l1, seq.batch, [0], rows, what="16k 100-chunks (sampled)")
    same = bits_equal(of, o1) and bits_equal(lf, l1)
    say(f"16k 100-chunks bit-equal to unchunked: {same}")


def test_decode_probe_batch_sizes_1_to_64():
    """A probe request (own seed, 20000-token context) at a varying position in
    batches of 1..64 requests with uniform [1, 32768] contexts and re-drawn
    page ids: its output bits never change."""
    ref = None
    for B in range(1, 65):
        pos = (B * 13 // 7) % B
        say(f"decode probe B={B} pos={pos}")
        b = W.decode_batch(B, seed=4, num_pages=131072, device=DEV,
                           probe=(pos, 20000, 40))
        out, lse = run_decode(b)
        o, l = out[pos].clone(), lse[pos].clone()
        if ref is None:
            ref = (o, l)
            assert_parity(out, lse, b, [pos], what="probe vs oracle")
        else:
            assert bits_equal(ref[0], o) and bits_equal(ref[1], l), f"probe differs at B={B}"


def test_decode_run_to_run():
    say("decode repeat B=32")
    b = W.decode_batch(32, seed=6, num_pages=131072, device=DEV)
    o1, l1 = run_decode(b)
    o2, l2 = run_decode(b)
    assert bits_equal(o1, o2) and bits_equal(l1, l2)


def _filler_requests(B, rng):
    """B short requests with their own seeds: some fresh prefills, some chunks
    over a cached prefix, some empty."""
    qo = rng.integers(0, 300, size=B)
    kv = qo + rng.integers(0, 600, size=B)
    return [W.Request(int(a), int(b), 9000 + 97 * B + i) for i, (a, b) in enumerate(zip(qo, kv))]


def test_prefill_probe_batch_sizes_1_to_64():
    """A probe prefill request (a 600-token chunk over a 900-token cached
    prefix, its own seed) at a varying position in batches of 1..64 seeded
    neighbours, with page ids re-drawn per batch: its out/lse bits never
    change, at the default split and at a split that merges partitions."""
    probe = W.Request(600, 1500, 4242)
    refs = {}
    for B in range(1, 65):
        pos = (B * 13 // 7) % B
        rng = np.random.Generator(np.random.PCG64(500 + B))
        reqs = _filler_requests(B, rng)
        reqs[pos] = probe
        b = W.make_batch(reqs, num_pages=8192, batch_seed=700 + B, device=DEV, **W.QWEN3_8B)
        for split in (4096, 512):
            say(f"prefill probe B={B} pos={pos} split={split}")
            out, lse = run_prefill(b, split=split)
            o, l = out[rows_of(b, pos)].clone(), lse[rows_of(b, pos)].clone()
            if split not in refs:
                refs[split] = (o, l)
                assert_parity(out, lse, b, [pos], what=f"prefill probe vs oracle split {split}")
            else:
                assert bits_equal(refs[split][0], o) and bits_equal(refs[split][1], l), \
                    f"prefill probe differs at B={B} split={split}"
