"""Plans destroyed while their work is still queued.

A plan takes a pinned work-list block from the library's pool when it is made
and gives it back on destroy; the block is handed out again only after the
device has passed the upload that read it. Here two plans of equal size but
different work lists alternate, each destroyed right after its run call is
enqueued, so a block handed out too early would give the next call the other
plan's list (both lists stay in bounds for either batch, so such a mistake
shows as wrong bits, not as a fault)."""
import numpy as np
import pytest
import torch

import invariant_paged_kv_amd as bia
import workloads as W
from gpu_util import bits_equal, page_table_dev, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _plan(b, mode, split):
    return bia.bia_plan_create(mode, b.qo_indptr, b.kv_indptr, b.page_table,
                               num_qo_heads=b.num_qo_heads, num_kv_heads=b.num_kv_heads,
                               head_dim=b.head_dim, num_pages=b.num_pages, split_size=split)


@pytest.mark.parametrize("mode", ["prefill", "decode"])
def test_destroy_while_queued(mode):
    say(f"plan pool: destroy while queued ({mode})")
    kw = dict(num_pages=4096, device=DEV, **W.QWEN3_8B)
    if mode == "prefill":
        # equal total tokens and pages, different items; no partial states
        a = W.make_batch([W.Request(1000, 1000, 701), W.Request(3000, 3000, 702)],
                         batch_seed=11, **kw)
        b = W.make_batch([W.Request(3000, 3000, 702), W.Request(1000, 1000, 701)],
                         batch_seed=12, **kw)
        m, split, fn = bia.BIA_MODE_PREFILL, bia.BIA_PREFILL_SPLIT, bia.bia_prefill_paged
    else:
        a = W.decode_batch(8, ctx_lens=[100, 2000, 40, 1500, 9, 2048, 700, 1200], seed=21,
                           num_pages=4096, device=DEV)
        b = W.decode_batch(8, ctx_lens=[1200, 700, 2048, 9, 1500, 40, 2000, 100], seed=22,
                           num_pages=4096, device=DEV)
        m, split, fn = bia.BIA_MODE_DECODE, bia.BIA_DECODE_SPLIT, bia.bia_decode_paged
    batches = (a, b)
    pts = [page_table_dev(x) for x in batches]
    refs = []
    for x, pt in zip(batches, pts):
        p = _plan(x, m, split)
        out = torch.empty_like(x.q)
        lse = torch.empty(x.q.shape[:2], dtype=torch.float32, device=DEV)
        ws = torch.empty(max(p.workspace_bytes, 256), dtype=torch.uint8, device=DEV)
        fn(p, x.q, x.k_pool, x.v_pool, pt, x.sm_scale, out, lse, ws)
        torch.cuda.synchronize()
        p.close()
        refs.append((out, lse))
    n = 24
    outs = [[torch.empty_like(x.q) for _ in range(n)] for x in batches]
    lses = [[torch.empty(x.q.shape[:2], dtype=torch.float32, device=DEV) for _ in range(n)]
            for x in batches]
    wss = [torch.empty(1 << 20, dtype=torch.uint8, device=DEV) for _ in range(2 * n)]
    for i in range(n):
        for k, (x, pt) in enumerate(zip(batches, pts)):
            p = _plan(x, m, split)
            assert p.workspace_bytes <= wss[0].numel()
            fn(p, x.q, x.k_pool, x.v_pool, pt, x.sm_scale, outs[k][i], lses[k][i],
               wss[2 * i + k])
            p.close()        # destroyed at once, its upload still queued
    torch.cuda.synchronize()
    for k in range(2):
        for i in range(n):
            assert bits_equal(outs[k][i], refs[k][0]), f"batch {k} call {i}: out differs"
            assert bits_equal(lses[k][i], refs[k][1]), f"batch {k} call {i}: lse differs"
