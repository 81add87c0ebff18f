"""Split sizes away from the defaults, against the float64 oracle.

The split is a plan argument (any positive multiple of the 64-key tile);
the oracle does not depend on it, so every split must meet the same
tolerance.

* Prefill at splits 8192 and 16384 over a 12000-token prefix: items whose
  tile loop runs up to 256 tiles, rows that span two partitions (8192) or
  one (16384, written directly without a merge), next to a request with no
  prefix.
* Decode at splits 64, 1024, 4096, 16384 and 32768 over contexts from 1 to
  17000 keys: up to 266 partition states folded per request (split 64), and
  requests that fit in one partition at the larger splits. Up to 16384 the
  decode runs on MFMA; 32768 is past its page list and runs the VALU decode
  at the same head dim."""
import pytest

import workloads as W
from gpu_util import assert_parity, run_decode, run_prefill, sample_rows, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("split", [8192, 16384])
def test_prefill_large_splits(split):
    reqs = [W.Request(700, 12700, 9101), W.Request(300, 300, 9102)]
    say(f"prefill split {split}: {[(r.qo_len, r.kv_len) for r in reqs]}")
    b = W.make_batch(reqs, num_pages=1024, batch_seed=9103, device=DEV, **W.QWEN3_8B)
    out, lse = run_prefill(b, split=split)
    rows = {0: sample_rows(700), 1: sample_rows(300)}
    assert_parity(out, lse, b, reqs=[0, 1], local_rows=rows, what=f"prefill split {split}")


@pytest.mark.parametrize("split", [64, 1024, 4096, 16384, 32768])
def test_decode_splits(split):
    ctx = [1, 63, 2049, 5000, 9000, 17000]
    say(f"decode split {split}: ctx {ctx}")
    b = W.decode_batch(len(ctx), ctx_lens=ctx, seed=31, num_pages=4096, device=DEV)
    out, lse = run_decode(b, split=split)
    assert_parity(out, lse, b, what=f"decode split {split}")


@pytest.mark.parametrize("heads", [dict(num_qo_heads=16, num_kv_heads=2, head_dim=64),
                                   dict(num_qo_heads=4, num_kv_heads=1, head_dim=64)],
                         ids=["hq16_hkv2_d64", "hq4_hkv1_d64"])
def test_decode_split_32768_head_dim_64(heads):
    """head_dim 64 past the MFMA decode's page list: the VALU decode."""
    ctx = [1, 63, 2049, 17000, 40000]
    say(f"decode split 32768 {heads}: ctx {ctx}")
    b = W.decode_batch(len(ctx), ctx_lens=ctx, seed=37, num_pages=8192, device=DEV, head=heads)
    out, lse = run_decode(b, split=32768)
    assert_parity(out, lse, b, what=f"decode split 32768 {heads}")
