"""Graph-capturable decode on the GPU. The device-planned decode keeps the
fixed split (the pages' runtime turns split-KV off under graph capture,
"[POC] Support deterministic inference", sglang PR #10417, Modifications), so
its out / lse bits equal those of the host-planned decode of the same split
size: run eagerly, and replayed from a captured HIP graph whose buffers get
new contents between replays. Invalid requests are flagged by the device
planner and come out as the empty state without touching the other rows."""
import numpy as np
import pytest
import torch

import invariant_paged_kv_amd as bia
import workloads as W
from gpu_util import assert_parity, bits_equal, run_decode, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def make_dg(b, max_batch, max_kv_len, capacity):
    return bia.bia_decode_graph_create(
        max_batch=max_batch, num_qo_heads=b.num_qo_heads, num_kv_heads=b.num_kv_heads,
        head_dim=b.head_dim, num_pages=b.num_pages, max_kv_len=max_kv_len,
        page_table_capacity=capacity)


def device_tables(b, capacity):
    """Device kv_indptr and a page table padded with zeros to the capacity."""
    ind = torch.as_tensor(b.kv_indptr, dtype=torch.int32, device=DEV)
    pt = torch.zeros(capacity, dtype=torch.int32, device=DEV)
    n = b.page_table.size
    pt[:n] = torch.as_tensor(b.page_table, dtype=torch.int32, device=DEV)
    return ind, pt


def run_graph_decode(dg, b, capacity, page_table=None):
    ind = torch.as_tensor(b.kv_indptr, dtype=torch.int32, device=DEV)
    pt = page_table if page_table is not None else device_tables(b, capacity)[1]
    out = torch.full_like(b.q, float("nan"))
    lse = torch.full(b.q.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(dg.workspace_bytes, dtype=torch.uint8, device=DEV)
    bia.bia_decode_graph_run(dg, b.batch, ind, b.q, b.k_pool, b.v_pool, pt, b.sm_scale,
                             out, lse, ws)
    torch.cuda.synchronize()
    return out, lse, bia.bia_decode_graph_read_flags(dg, ws, b.batch)


@pytest.mark.parametrize("head", [W.QWEN3_8B, dict(num_qo_heads=8, num_kv_heads=1,
                                                   head_dim=64)])
def test_eager_equals_planned(head):
    """Lengths around the 2048-key partition edges, the maximum, and one key."""
    ctx = [1, 2, 17, 2047, 2048, 2049, 4096, 4097, 6000, 16384, 100, 12345]
    say(f"graph decode eager vs planned, heads {head}")
    b = W.decode_batch(len(ctx), seed=61, num_pages=4096, device=DEV, ctx_lens=ctx, head=head)
    o_ref, l_ref = run_decode(b)
    dg = make_dg(b, max_batch=16, max_kv_len=16384, capacity=4096)   # 3080 pages used
    out, lse, flags = run_graph_decode(dg, b, 4096)
    dg.close()
    assert (flags == 0).all(), flags
    assert bits_equal(out, o_ref) and bits_equal(lse, l_ref)
    assert_parity(out, lse, b, [0, 3, 5, 9], what="graph decode")


def test_graph_replay_equals_planned():
    """One capture, three replays with new lengths, pages, queries and pools;
    eager work and synchronisations between the replays."""
    B, cap, max_kv, pool = 8, 8192, 16384, 8192
    b0 = W.decode_batch(B, seed=71, num_pages=pool, device=DEV, max_ctx=max_kv)
    dg = make_dg(b0, B, max_kv, cap)
    ind = torch.zeros(B + 1, dtype=torch.int32, device=DEV)
    pt = torch.zeros(cap, dtype=torch.int32, device=DEV)
    q = torch.empty_like(b0.q)
    kpool = torch.empty_like(b0.k_pool)
    vpool = torch.empty_like(b0.v_pool)
    out = torch.empty_like(b0.q)
    lse = torch.empty(b0.q.shape[:2], dtype=torch.float32, device=DEV)
    ws = torch.empty(dg.workspace_bytes, dtype=torch.uint8, device=DEV)

    def load(b):
        d_ind, d_pt = device_tables(b, cap)
        ind.copy_(d_ind)
        pt.copy_(d_pt)
        q.copy_(b.q)
        kpool.copy_(b.k_pool)
        vpool.copy_(b.v_pool)

    def call():
        bia.bia_decode_graph_run(dg, B, ind, q, kpool, vpool, pt, b0.sm_scale, out, lse, ws)

    load(b0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("graph decode: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for seed in (72, 73, 74):
        b = W.decode_batch(B, seed=seed, num_pages=pool, device=DEV, max_ctx=max_kv)
        load(b)
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"graph decode: replay with seed {seed}, ctx {b.kv_lens().tolist()}")
        g.replay()
        torch.cuda.synchronize()
        o_ref, l_ref = run_decode(b)
        assert bits_equal(out, o_ref) and bits_equal(lse, l_ref), f"replay seed {seed}"
    flags = bia.bia_decode_graph_read_flags(dg, ws, B)
    assert (flags == 0).all(), flags
    del g
    dg.close()


def test_invalid_requests_are_flagged():
    """kv_len past the capacity (flag 1), a page id outside the pool (4) and
    pages past the table capacity (2): those rows are the empty state, the
    valid row keeps its bits."""
    ctx = [300, 5000, 64, 700]
    b = W.decode_batch(len(ctx), seed=81, num_pages=1024, device=DEV, ctx_lens=ctx)
    pages = (np.asarray(ctx) + 15) // 16          # 19, 313, 4, 44
    cap = int(pages[:3].sum() + 20)               # request 3 runs past it
    dg = make_dg(b, max_batch=4, max_kv_len=4096, capacity=cap)
    _, pt = device_tables(b, int(pages.sum()))
    pt = pt[:cap].clone()
    pt[int(pages[:2].sum())] = b.num_pages        # request 2's first page id
    say("graph decode: invalid requests")
    out, lse, flags = run_graph_decode(dg, b, cap, page_table=pt)
    dg.close()
    assert flags.tolist() == [0, 1, 4, 2], flags
    for r in (1, 2, 3):
        assert torch.count_nonzero(out[r].float()) == 0
        assert torch.isneginf(lse[r]).all()
    alone = W.decode_batch(1, seed=81, num_pages=1024, device=DEV, ctx_lens=ctx[:1])
    o1, l1 = run_decode(alone)
    assert bits_equal(out[:1], o1) and bits_equal(lse[:1], l1)


def test_device_plan_matches_host_plan():
    """The device planner's work list is the host planner's (all fields but
    the partial-state slot) in the host's launch order: whole partitions in
    (request, kv head, partition) order, partial last partitions longest
    first, then the empty slots."""
    ctx = [4096, 1, 2048, 2049, 6000, 16384, 100, 12345, 4095]
    b = W.decode_batch(len(ctx), seed=91, num_pages=4096, device=DEV, ctx_lens=ctx)
    max_batch, max_kv, cap = 12, 16384, 4096
    dg = make_dg(b, max_batch, max_kv, cap)
    ind, pt = device_tables(b, cap)
    out = torch.empty_like(b.q)
    lse = torch.empty(b.q.shape[:2], dtype=torch.float32, device=DEV)
    ws = torch.zeros(dg.workspace_bytes, dtype=torch.uint8, device=DEV)
    say("graph decode: device plan vs host plan")
    bia.bia_decode_graph_run(dg, b.batch, ind, b.q, b.k_pool, b.v_pool, pt, b.sm_scale, out,
                             lse, ws)
    torch.cuda.synchronize()
    max_splits = (max_kv + 2047) // 2048
    off_items = (max_batch * 4 + 255) // 256 * 256
    n = b.batch * b.num_kv_heads * max_splits
    dev_items = ws[off_items: off_items + n * 32].view(torch.int32).view(n, 8).cpu().numpy()
    dg.close()
    plan = bia.bia_plan_create(bia.BIA_MODE_DECODE, b.qo_indptr, b.kv_indptr, b.page_table,
                               num_qo_heads=b.num_qo_heads, num_kv_heads=b.num_kv_heads,
                               head_dim=b.head_dim, num_pages=b.num_pages, split_size=2048)
    host_items = plan.items()
    plan.close()
    live = dev_items[dev_items[:, 1] > 0]
    assert len(live) == len(host_items)
    key = lambda a: sorted(map(tuple, a[:, :7].tolist()))
    assert key(live) == key(host_items)
    # the same launch order as the host plan
    assert (dev_items[:len(live), :7] == np.asarray(host_items)[:, :7]).all()
    # order: whole partitions, then partial ones, then the empty slots
    n_live = len(live)
    assert (dev_items[n_live:, 1] == 0).all()
    lens = np.minimum(live[:, 3] - live[:, 6], 2048)
    whole = lens == 2048
    assert not whole[np.argmax(~whole):].any() if (~whole).any() else True
    # partial partitions longest first (in 64-key tiles), as the host plan sorts them
    tiles = (lens[~whole] + 63) // 64
    assert (np.diff(tiles) <= 0).all(), "partial partitions are not launched longest first"
