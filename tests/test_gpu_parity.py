"""GPU path vs the float64 CPU oracle, element by element on the same seeded
inputs: max abs error <= 2e-2 on bf16 outputs and <= 1e-3 on lse.

Small cases compare every row; the full-size workloads (in the launch
configuration the benchmark times) compare a fixed row sample: the first and
last 128 query tokens of each request and every 61st token, all heads."""
import math

import numpy as np
import pytest
import torch

import invariant_paged_kv_amd as bia
import oracle
import oracle_pins
import workloads as W
from gpu_util import (LSE_TOL, OUT_TOL, assert_parity, bits_equal, run_decode,
                      run_prefill, sample_rows, say)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_tiny_prefill_all_rows():
    say("tiny prefill, split 4096")
    b = W.tiny_prefill(device=DEV)
    out, lse = run_prefill(b)
    assert_parity(out, lse, b, what="tiny split 4096")


@pytest.mark.parametrize("split", [64, 128, 192])
def test_tiny_prefill_small_splits_merge(split):
    say(f"tiny prefill, split {split}")
    b = W.tiny_prefill(device=DEV)
    out, lse = run_prefill(b, split=split)
    assert_parity(out, lse, b, what=f"tiny split {split}")


def test_three_token_hand_example():
    say("3-token hand example, D padded to 64")
    b = oracle_pins.three_token_batch(head_dim=64).to(DEV)
    out, lse = run_prefill(b)
    gold = oracle_pins.load_three_token_golden()
    o = out[:, 0, :2].double().cpu().numpy()
    assert np.max(np.abs(o - gold[:, 1:3])) <= OUT_TOL
    assert np.max(np.abs(lse[:, 0].double().cpu().numpy() - gold[:, 3])) <= LSE_TOL
    assert torch.all(out[:, 0, 2:] == 0)
    # row 0 has one key: out is v_0 exactly
    assert out[0, 0, 0].item() == 1.0 and out[0, 0, 1].item() == 0.0


def test_one_key_is_exact():
    """kv_len = 1 gives out = v_0 bit for bit (p = 1, l = 1)."""
    say("one-key exactness, prefill and decode")
    reqs = [W.Request(1, 1, 301), W.Request(1, 1, 302)]
    b = W.make_batch(reqs, num_pages=64, batch_seed=5, device=DEV, keep_seq=True,
                     **W.QWEN3_8B)
    for out, _ in (run_prefill(b), run_decode(b)):
        for r in range(2):
            v0 = b.v_seq[r][0].to(DEV)  # [Hkv, D]
            expect = v0.repeat_interleave(4, dim=0)
            assert bits_equal(out[r], expect)


@pytest.mark.parametrize("heads", [
    dict(num_qo_heads=32, num_kv_heads=8, head_dim=128),
    dict(num_qo_heads=8, num_kv_heads=8, head_dim=128),
    dict(num_qo_heads=16, num_kv_heads=8, head_dim=64),
    dict(num_qo_heads=16, num_kv_heads=2, head_dim=128),
    dict(num_qo_heads=4, num_kv_heads=1, head_dim=64),
], ids=lambda h: f"hq{h['num_qo_heads']}_hkv{h['num_kv_heads']}_d{h['head_dim']}")
@pytest.mark.parametrize("split", [256, 4096])
def test_ragged_prefill(heads, split):
    """Ragged mix: empty query, single token, prefix + chunk, fresh prefill,
    lengths off the page and tile sizes."""
    say(f"ragged prefill {heads} split {split}")
    reqs = [W.Request(0, 20, 401), W.Request(1, 1, 402), W.Request(77, 300, 403),
            W.Request(129, 129, 404), W.Request(1, 1000, 405), W.Request(500, 1100, 406)]
    b = W.make_batch(reqs, num_pages=512, batch_seed=8, device=DEV, **heads)
    out, lse = run_prefill(b, split=split)
    assert_parity(out, lse, b, what=f"ragged {heads} split {split}")


@pytest.mark.parametrize("heads", [
    dict(num_qo_heads=32, num_kv_heads=8, head_dim=128),
    dict(num_qo_heads=8, num_kv_heads=8, head_dim=128),
    dict(num_qo_heads=16, num_kv_heads=2, head_dim=64),
    dict(num_qo_heads=16, num_kv_heads=4, head_dim=128),
    dict(num_qo_heads=64, num_kv_heads=8, head_dim=128),
    dict(num_qo_heads=16, num_kv_heads=8, head_dim=128),
], ids=lambda h: f"hq{h['num_qo_heads']}_hkv{h['num_kv_heads']}_d{h['head_dim']}")
def test_decode_small(heads):
    say(f"decode small {heads}")
    ctx = [1, 2, 15, 16, 17, 31, 33, 100, 2047, 2048, 2049, 4096, 5000, 9999]
    b = W.decode_batch(len(ctx), ctx_lens=ctx, num_pages=4096, device=DEV, head=heads)
    out, lse = run_decode(b)
    assert_parity(out, lse, b, what=f"decode small {heads}")


def test_qwen_prefill_full_size():
    """8 x 4096 tokens, 32/8 heads, D 128, 64K-page pool, split 4096."""
    say("Qwen3-8B prefill 8 x 4096")
    b = W.qwen_prefill(device=DEV)
    out, lse = run_prefill(b)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    reqs = [0, 5]
    rows = {r: sample_rows(4096) for r in reqs}
    assert_parity(out, lse, b, reqs, rows, what="qwen prefill (sampled)")


def test_decode_full_size_b64():
    """64 requests, contexts uniform in [1, 32768], 128K-page pool, split 2048."""
    say("decode B=64, ctx U[1, 32768]")
    b = W.decode_batch(64, device=DEV)
    out, lse = run_decode(b)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    kv = b.kv_lens()
    reqs = sorted(set([int(np.argmax(kv)), int(np.argmin(kv))] + list(range(0, 64, 9))))
    assert_parity(out, lse, b, reqs, what="decode B=64 (sampled requests)")


def test_mixed_long_context_step():
    """Last 16384-token chunk of a 65536-token prefill, and 128 decodes with
    lognormal contexts (median 4096, sigma 1, cap 131072)."""
    say("mixed: prefill chunk 49152..65536 + 128 decodes")
    seq = W.make_sequence(65536, seed=5, num_pages=8192, device=DEV)
    ch = seq.chunk(49152, 65536)
    out, lse = run_prefill(ch)
    rows = {0: sample_rows(16384, edge=64, every=509)}
    assert_parity(out, lse, ch, [0], rows, what="mixed prefill chunk 4 (sampled)")
    ctx = W.mixed_decode_lengths()
    d = W.decode_batch(128, ctx_lens=ctx, seed=5, num_pages=131072, device=DEV,
                       max_ctx=131072)
    dout, dlse = run_decode(d)
    reqs = sorted(set([int(np.argmax(ctx))] + list(range(0, 128, 16))))
    assert_parity(dout, dlse, d, reqs, what="mixed decodes (sampled)")


@pytest.mark.parametrize("D", [64, 128])
def test_merge_states(D):
    say(f"bia_merge_states D={D}")
    g = torch.Generator().manual_seed(10 + D)
    H, n_rows = 3, 7
    counts = [0, 1, 2, 5, 3, 1, 4]
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    n = int(indptr[-1])
    v = torch.randn(n, H, D, generator=g)
    s = torch.randn(n, H, generator=g) * 3
    s[2, 1] = float("-inf")                       # an empty state in a live row
    s[indptr[5]:indptr[6], :] = float("-inf")     # a row of only empty states
    v[indptr[5]:indptr[6]] = 0
    out = torch.empty(n_rows, H, D, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(n_rows, H, dtype=torch.float32, device=DEV)
    bia.bia_merge_states(v.to(DEV), s.to(DEV), torch.as_tensor(indptr, device=DEV), out, lse)
    torch.cuda.synchronize()
    ro, rl = oracle.merge_states(v.double().numpy(), s.double().numpy(), indptr)
    o = out.double().cpu().numpy()
    l = lse.double().cpu().numpy()
    assert np.max(np.abs(o - ro)) <= OUT_TOL
    fin = np.isfinite(rl)
    assert np.all(np.isneginf(l[~fin])) and np.all(o[~fin] == 0)
    assert np.max(np.abs(l[fin] - rl[fin])) <= LSE_TOL
    # a row with one live state reproduces it exactly
    assert bits_equal(out[1].cpu(), v[indptr[1]].to(torch.bfloat16))


@pytest.mark.parametrize("heads", [W.QWEN3_8B, dict(num_qo_heads=4, num_kv_heads=1, head_dim=64)],
                         ids=["hq32_hkv8_d128", "hq4_hkv1_d64"])
@pytest.mark.parametrize("split", [256, 4096])
def test_rising_logits_prefill(split, heads):
    """Logits that climb along the sequence make a row's running max rise
    again and again (many raises after the first tile, with O and l already
    holding earlier keys); the partitions of the 4500-key request merge states
    whose lse differ by tens of units."""
    say(f"rising logits prefill, split {split}, {heads}")
    b = W.rising_batch([1000, 300, 37], [1000, 4500, 37], seed=61, num_pages=512,
                       device=DEV, **heads)
    out, lse = run_prefill(b, split=split)
    assert_parity(out, lse, b, what=f"rising prefill split {split}")


def test_rising_logits_decode():
    say("rising logits decode")
    ctx = [1, 100, 2048, 2049, 5000, 9000]
    b = W.rising_batch([1] * len(ctx), ctx, seed=62, num_pages=2048, device=DEV,
                       **W.QWEN3_8B)
    out, lse = run_decode(b)
    assert_parity(out, lse, b, what="rising decode")
