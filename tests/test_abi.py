"""C-ABI library on the CPU: it loads, exports what bia.h declares, validates
its arguments before any launch, and plans work lists whose layout depends on
each request's own lengths only. No kernel runs here."""
import ctypes
import os
import re

import numpy as np
import pytest

import invariant_paged_kv_amd as bia
from invariant_paged_kv_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bia.h")

QWEN = dict(num_qo_heads=32, num_kv_heads=8, head_dim=128)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bia_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = bia.load_library()
    names = declared_functions()
    assert "bia_prefill_paged" in names and "bia_merge_states" in names
    for name in names:
        assert hasattr(lib, name), f"libbia.so does not export {name}"


def test_python_binding_has_every_entry_point():
    """The binding keeps the C names of the calls a user makes."""
    for name in ["bia_plan_create", "bia_plan_destroy", "bia_plan_workspace_bytes",
                 "bia_prefill_paged", "bia_decode_paged", "bia_merge_states",
                 "bia_prefill_chunk_align", "bia_last_error", "bia_append_paged_kv",
                 "bia_decode_graph_create", "bia_decode_graph_destroy",
                 "bia_decode_graph_workspace_bytes", "bia_decode_graph_run",
                 "bia_decode_graph_read_flags", "bia_mla_prefill_paged",
                 "bia_mla_decode_paged", "bia_decode_paged_static"]:
        assert name in declared_functions()
        assert callable(getattr(bia, name)), name


def test_chunk_align_is_128():
    assert bia.bia_prefill_chunk_align() == 128


def plan(mode=bia.BIA_MODE_PREFILL, qo=(0, 100, 400), kv=(0, 100, 400), pt=None,
         heads=dict(num_qo_heads=4, num_kv_heads=1, head_dim=64), num_pages=64,
         split=4096, flags=0):
    if pt is None:
        kvl = np.diff(kv)
        pt = np.arange(int(((kvl + 15) // 16).sum()))
    return bia.bia_plan_create(mode, qo, kv, pt, num_pages=num_pages, split_size=split,
                               flags=flags, **heads)


@pytest.mark.parametrize("kwargs,status", [
    (dict(qo=(0, 5, 3), kv=(0, 10, 20)), "BIA_ERR_SHAPE"),        # qo decreases
    (dict(qo=(1, 5), kv=(0, 10)), "BIA_ERR_SHAPE"),               # does not start at 0
    (dict(qo=(0, 11), kv=(0, 10)), "BIA_ERR_SHAPE"),              # qo_len > kv_len
    (dict(qo=(0, 1), kv=(0, 10), pt=[0]), None),                  # fine (1 page)
    (dict(qo=(0, 1), kv=(0, 10), pt=[64]), "BIA_ERR_PAGE_RANGE"),
    (dict(qo=(0, 1), kv=(0, 10), pt=[-1]), "BIA_ERR_PAGE_RANGE"),
    (dict(split=100), "BIA_ERR_INVALID_ARG"),                     # not a multiple of 64
    (dict(split=0), "BIA_ERR_INVALID_ARG"),
    (dict(heads=dict(num_qo_heads=4, num_kv_heads=1, head_dim=96)), "BIA_ERR_UNSUPPORTED"),
    (dict(heads=dict(num_qo_heads=6, num_kv_heads=4, head_dim=64)), "BIA_ERR_SHAPE"),
    (dict(heads=dict(num_qo_heads=48, num_kv_heads=3, head_dim=64)), "BIA_ERR_UNSUPPORTED"),
    (dict(mode=bia.BIA_MODE_DECODE), "BIA_ERR_SHAPE"),            # decode needs qo_len 1
    (dict(mode=7), "BIA_ERR_INVALID_ARG"),
    (dict(flags=0x4), "BIA_ERR_INVALID_ARG"),                     # unknown flag
    # strict chunk alignment: starts at 0 and 128 pass, 100 is rejected
    (dict(qo=(0, 100, 400), kv=(0, 100, 400), flags=1), None),
    (dict(qo=(0, 172), kv=(0, 300), flags=1), None),
    (dict(qo=(0, 200), kv=(0, 300), flags=1), "BIA_ERR_INVALID_ARG"),
    (dict(qo=(0, 200), kv=(0, 300), flags=0), None),
    (dict(mode=bia.BIA_MODE_DECODE, qo=(0, 1), kv=(0, 300), flags=1), None),
])
def test_plan_validation(kwargs, status):
    if status is None:
        plan(**kwargs).close()
        return
    with pytest.raises(bia.BiaError) as e:
        plan(**kwargs)
    assert str(e.value).startswith(status), str(e.value)
    assert bia.bia_last_error()
    if kwargs.get("flags") == 1:
        assert "aligned to 128 tokens" in bia.bia_last_error()


def test_null_pointers_rejected_before_anything_runs():
    lib = bia.load_library()
    h = ctypes.c_void_p()
    assert lib.bia_plan_create(0, None, None, None, 2, 4, 1, 64, 16, 64, 4096, 0,
                               ctypes.byref(h)) == 1
    assert lib.bia_plan_create(0, None, None, None, 0, 4, 1, 64, 16, 64, 4096, 0,
                               None) == 1
    assert lib.bia_append_paged_kv(None, None, None, None, None, None, None, 0, None) == 1
    # run calls with a NULL plan fail in the argument check (no HIP call)
    assert lib.bia_prefill_paged(None, None, None, None, None, 1.0, None, None, None, 0,
                                 None) == 1
    assert lib.bia_decode_paged(None, None, None, None, None, 1.0, None, None, None, 0,
                                None) == 1
    assert lib.bia_merge_states(None, None, None, 4, 2, 96, None, None, None) == 5
    assert lib.bia_merge_states(None, None, None, 4, 2, 64, None, None, None) == 1
    assert lib.bia_merge_states(None, None, None, 0, 2, 64, None, None, None) == 0
    lib.bia_plan_destroy(None)


def test_empty_batch_plan():
    p = bia.bia_plan_create(bia.BIA_MODE_PREFILL, [0], [0], None, num_pages=0,
                            split_size=4096, **QWEN)
    assert p.num_items == 0 and p.num_states == 0
    p.close()


def test_run_rejects_wrong_mode_and_small_workspace():
    lib = bia.load_library()
    p = plan()
    # decode call on a prefill plan: rejected in the argument check
    st = lib.bia_decode_paged(ctypes.c_void_p(p.handle), None, None, None, None, 1.0, None,
                              None, None, 0, None)
    assert st == 1 and "mode" in bia.bia_last_error()
    dummy = ctypes.c_void_p(256)
    st = lib.bia_prefill_paged(ctypes.c_void_p(p.handle), dummy, dummy, dummy, dummy, 1.0,
                               dummy, None, dummy, p.workspace_bytes - 1, None)
    assert st == 4, bia.bia_last_error()
    st = lib.bia_prefill_paged(ctypes.c_void_p(p.handle), dummy, dummy, dummy, dummy,
                               float("nan"), dummy, None, dummy, p.workspace_bytes, None)
    assert st == 1
    p.close()


# ------------------------------------------------------- latent (MLA) plans --

MLA = dict(num_kv_heads=1, head_dim=bia.BIA_MLA_QK_DIM)


@pytest.mark.parametrize("heads,status", [
    (dict(num_qo_heads=16, **MLA), None),
    (dict(num_qo_heads=128, **MLA), None),
    (dict(num_qo_heads=8, **MLA), None),
    (dict(num_qo_heads=12, **MLA), "BIA_ERR_UNSUPPORTED"),       # not a power of 2
    (dict(num_qo_heads=256, **MLA), "BIA_ERR_UNSUPPORTED"),
    (dict(num_qo_heads=16, num_kv_heads=2, head_dim=576), "BIA_ERR_SHAPE"),
    (dict(num_qo_heads=16, num_kv_heads=1, head_dim=128), "BIA_ERR_UNSUPPORTED"),
])
def test_mla_plan_validation(heads, status):
    kw = dict(heads=heads, flags=bia.BIA_PLAN_MLA)
    if status is None:
        plan(**kw).close()
        return
    with pytest.raises(bia.BiaError) as e:
        plan(**kw)
    assert str(e.value).startswith(status), str(e.value)


def test_mla_split_limit():
    """The item's page list is held on chip: MLA splits above
    BIA_MLA_MAX_SPLIT are rejected."""
    heads = dict(num_qo_heads=16, **MLA)
    plan(heads=heads, flags=bia.BIA_PLAN_MLA, split=bia.BIA_MLA_MAX_SPLIT).close()
    with pytest.raises(bia.BiaError) as e:
        plan(heads=heads, flags=bia.BIA_PLAN_MLA, split=bia.BIA_MLA_MAX_SPLIT + 64)
    assert str(e.value).startswith("BIA_ERR_UNSUPPORTED")


def test_mla_plan_without_flag_rejects_576():
    with pytest.raises(bia.BiaError) as e:
        plan(heads=dict(num_qo_heads=16, **MLA))
    assert str(e.value).startswith("BIA_ERR_UNSUPPORTED")


@pytest.mark.parametrize("hq", [16, 128])
def test_mla_items_cover_every_head_and_token(hq):
    """Items of a latent plan: 128-row tiles of 128 / min(Hq, 128) tokens, one
    per head block, so every (token, q head) row sits in exactly one tile of
    each partition it needs; partial states hold 512 dims."""
    p = plan(qo=(0, 100, 400), kv=(0, 100, 700), heads=dict(num_qo_heads=hq, **MLA),
             flags=bia.BIA_PLAN_MLA, split=256)
    hb = min(hq, 128)
    T = 128 // hb
    its = items_of(p)
    assert max(it["n_tok"] for it in its) == T
    assert {it["kv_head"] for it in its} == set(range(hq // hb))
    rows = {}
    for it in its:
        for t in range(it["n_tok"]):
            for j in range(hb):
                key = (it["q_row0"] + t, it["kv_head"] * hb + j)
                rows.setdefault(key, []).append(it["kv_begin"])
    assert len(rows) == 400 * hq
    for (row, h), parts in rows.items():
        # request 0: rows 0..99 at positions 0..99; request 1: rows 100..399
        # at positions 300..599; a row's tile reaches the last position of
        # its T-token tile (tiles start at the request's first row)
        base, first_pos, kv_len = (0, 0, 100) if row < 100 else (100, 300, 600)
        off = row - base
        tile_last = min(first_pos + off // T * T + T - 1, kv_len - 1)
        assert sorted(parts) == [256 * k for k in range(tile_last // 256 + 1)]
    assert p.workspace_bytes >= p.num_states * (512 + 1) * 4


def test_mla_plan_rejected_by_the_other_calls():
    lib = bia.load_library()
    p = plan(heads=dict(num_qo_heads=16, **MLA), flags=bia.BIA_PLAN_MLA)
    g = plan()
    dummy = ctypes.c_void_p(256)
    st = lib.bia_prefill_paged(ctypes.c_void_p(p.handle), dummy, dummy, dummy, dummy, 1.0,
                               dummy, None, dummy, p.workspace_bytes, None)
    assert st == 1 and "MLA" in bia.bia_last_error()
    st = lib.bia_mla_prefill_paged(ctypes.c_void_p(g.handle), dummy, dummy, dummy, 1.0,
                                   dummy, None, dummy, g.workspace_bytes, None)
    assert st == 1 and "BIA_PLAN_MLA" in bia.bia_last_error()
    st = lib.bia_mla_decode_paged(ctypes.c_void_p(p.handle), dummy, dummy, dummy, 1.0,
                                  dummy, None, dummy, p.workspace_bytes, None)
    assert st == 1 and "mode" in bia.bia_last_error()
    st = lib.bia_append_paged_kv(ctypes.c_void_p(p.handle), dummy, dummy, dummy, dummy,
                                 dummy, dummy, p.workspace_bytes, None)
    assert st == 5
    p.close()
    g.close()


# ------------------------------------------------------------ work lists ---

FIELDS = ["q_row0", "n_tok", "pos0", "kv_len", "page_off", "kv_head", "kv_begin", "state"]


def items_of(p):
    """The plan's work items in launch order, without the empty items that pad
    the prefill's per-XCD lists."""
    return [dict(zip(FIELDS, map(int, row))) for row in p.items() if row[1] > 0]


def item_tiles(it, split):
    last = it["pos0"] + it["n_tok"] - 1
    end = min(it["kv_begin"] + split, last + 1)
    return -(-(end - it["kv_begin"]) // 64)


@pytest.mark.parametrize("reqs,heads,split", [
    (dict(qo=(0, 4096, 8192), kv=(0, 4096, 8192)), QWEN, 4096),       # 16 pairs
    (dict(qo=(0, 1000), kv=(0, 3000)), dict(num_qo_heads=4, num_kv_heads=1, head_dim=64),
     1024),                                                            # 1 pair, shared out
    (dict(qo=(0, 5, 905, 1000, 3000), kv=(0, 5, 2000, 2095, 9000)), QWEN, 4096),
])
def test_prefill_launch_order_is_xcd_interleaved(reqs, heads, split):
    """Launch index 8 s + x runs on XCD x. Every item appears once; the
    per-XCD lists carry near-equal work (within the largest unit); on each
    XCD the items of one (request, kv head) pair are contiguous unless pairs
    were shared out; padding is empty items only."""
    p = plan(heads=heads, split=split, num_pages=4096, **reqs)
    rows = p.items()
    ref = plan(heads=heads, split=split, num_pages=4096, **reqs)
    real = [tuple(map(int, r)) for r in rows if r[1] > 0]
    assert len(set(real)) == len(real)
    assert all(tuple(r) == (0, 0, 0, 0, 0, 0, 0, -1) for r in rows if r[1] == 0)
    assert sorted(real) == sorted(tuple(map(int, r)) for r in ref.items() if r[1] > 0)
    xcd_work = [0] * 8
    xcd_pairs = [[] for _ in range(8)]
    for i, r in enumerate(rows):
        it = dict(zip(FIELDS, map(int, r)))
        if it["n_tok"] == 0:
            continue
        xcd_work[i % 8] += item_tiles(it, split)
        pair = (it["kv_len"], it["page_off"], it["kv_head"])
        if not xcd_pairs[i % 8] or xcd_pairs[i % 8][-1] != pair:
            xcd_pairs[i % 8].append(pair)
    n_pairs = len({(it["page_off"], it["kv_head"]) for it in items_of(p)})
    assert max(xcd_work) - min(xcd_work) <= max(xcd_work) // 2 + 64
    if n_pairs >= 32:
        for seq in xcd_pairs:          # each pair visited once per XCD
            assert len(seq) == len(set(seq))


def request_layout(p, q_row0, kv_head=0):
    """Items of the request whose first query row is q_row0, as
    (tile token offset, n_tok, pos0, kv_begin), sorted."""
    out = []
    for it in items_of(p):
        if it["kv_head"] == kv_head and it["q_row0"] >= q_row0:
            out.append(it)
    return out


def test_tiny_prefill_item_count_and_tiles():
    p = plan()
    its = items_of(p)
    # group 4 -> 32 tokens per tile: ceil(100/32) + ceil(300/32) = 4 + 10
    assert len(its) == 14
    assert all(it["state"] == -1 for it in its)  # one partition each at split 4096
    assert max(it["n_tok"] for it in its) == 32
    tok = sorted((it["q_row0"], it["n_tok"]) for it in its)
    covered = []
    for r0, n in tok:
        covered.extend(range(r0, r0 + n))
    assert covered == list(range(400))


@pytest.mark.parametrize("split", [64, 128, 4096])
def test_partitions_anchor_at_key_zero(split):
    p = plan(split=split)
    for it in items_of(p):
        assert it["kv_begin"] % split == 0
        last = it["pos0"] + it["n_tok"] - 1
        assert it["kv_begin"] <= last  # never an item with no visible key
    # every (tile, head) covers partitions 0..floor(last/split) exactly once
    seen = {}
    for it in items_of(p):
        key = (it["q_row0"], it["kv_head"])
        seen.setdefault(key, []).append(it["kv_begin"] // split)
    for (r0, h), parts in seen.items():
        its = [i for i in items_of(p) if i["q_row0"] == r0 and i["kv_head"] == h]
        last = its[0]["pos0"] + its[0]["n_tok"] - 1
        assert sorted(parts) == list(range(last // split + 1))


def test_request_layout_independent_of_batch():
    """A request's items (relative to its own rows) are the same alone and in
    a batch with others, in any position."""
    def rel(p, r0, base_page):
        return sorted((it["q_row0"] - r0, it["n_tok"], it["pos0"], it["kv_len"],
                       it["page_off"] - base_page, it["kv_head"], it["kv_begin"])
                      for it in items_of(p) if r0 <= it["q_row0"] < r0 + 1000
                      and it["kv_len"] == 1000)
    alone = plan(qo=(0, 1000), kv=(0, 1000), split=256, heads=QWEN, num_pages=4096)
    mixed = plan(qo=(0, 7, 1007, 1050), kv=(0, 33, 1033, 1500), split=256, heads=QWEN,
                 num_pages=4096)
    assert rel(alone, 0, 0) == rel(mixed, 7, 3)


def test_on_grid_chunk_tiles_are_unchunked_tiles():
    """A chunk starting on the 128-token grid cuts q tiles exactly where the
    unchunked call does (same pos0 / n_tok for every tile)."""
    full = plan(qo=(0, 16384), kv=(0, 16384), split=4096, heads=QWEN, num_pages=1024)
    tiles_full = {(it["pos0"], it["n_tok"], it["kv_begin"]) for it in items_of(full)}
    tiles_chunks = set()
    for c in range(64):
        ch = plan(qo=(0, 256), kv=(0, 256 * (c + 1)), split=4096, heads=QWEN,
                  num_pages=1024)
        tiles_chunks |= {(it["pos0"], it["n_tok"], it["kv_begin"]) for it in items_of(ch)}
    assert tiles_chunks == tiles_full


def test_decode_items_and_states():
    kv = np.array([1, 2048, 2049, 5000])
    kvp = np.concatenate([[0], np.cumsum(kv)])
    p = plan(mode=bia.BIA_MODE_DECODE, qo=np.arange(5), kv=kvp, split=2048, heads=QWEN,
             num_pages=4096)
    its = items_of(p)
    n_splits = [1, 1, 2, 3]
    assert len(its) == 8 * sum(n_splits)
    # requests with one partition write directly; the others use g = 4 states
    # per partition per kv head
    assert p.num_states == 8 * 4 * (2 + 3)
    for it in its:
        r = it["q_row0"]
        assert it["n_tok"] == 1 and it["pos0"] == kv[r] - 1 and it["kv_len"] == kv[r]
        assert (it["state"] == -1) == (n_splits[r] == 1)


def test_workspace_grows_with_states():
    a = plan(qo=(0, 1000), kv=(0, 1000), split=4096, heads=QWEN, num_pages=4096)
    b = plan(qo=(0, 1000), kv=(0, 1000), split=128, heads=QWEN, num_pages=4096)
    assert a.num_states == 0 and b.num_states > 0
    assert b.workspace_bytes >= b.num_states * (128 + 1) * 4
    assert a.workspace_bytes % 256 == 0 and b.workspace_bytes > a.workspace_bytes


def test_append_items_in_workspace():
    """The plan's uploaded blob grows by one 16-byte append item per 16 new
    tokens of each request."""
    a = plan(qo=(0, 16), kv=(0, 16))
    b = plan(qo=(0, 17), kv=(0, 17))
    c = plan(qo=(0, 0, 1), kv=(0, 20, 21))
    assert a.workspace_bytes >= 2 * 32 + 16     # 1 tile item (g=4: 32 tokens) + 1 append
    assert b.workspace_bytes >= 32 + 2 * 16     # 1 tile item + 2 appends
    assert c.workspace_bytes >= 32 + 16


# ----------------------------------------------------- graph-capturable decode --

GRAPH = dict(max_batch=64, num_qo_heads=32, num_kv_heads=8, head_dim=128, num_pages=1024,
             max_kv_len=32768, page_table_capacity=4096, split_size=2048)


@pytest.mark.parametrize("change,status", [
    ({}, None),
    (dict(max_batch=0), "BIA_ERR_INVALID_ARG"),
    (dict(max_kv_len=0), "BIA_ERR_INVALID_ARG"),
    (dict(page_table_capacity=-1), "BIA_ERR_INVALID_ARG"),
    (dict(split_size=100), "BIA_ERR_INVALID_ARG"),
    (dict(head_dim=96), "BIA_ERR_UNSUPPORTED"),
    (dict(num_qo_heads=48, num_kv_heads=3), "BIA_ERR_UNSUPPORTED"),
    (dict(num_qo_heads=6, num_kv_heads=4), "BIA_ERR_SHAPE"),
    (dict(page_size=32), "BIA_ERR_UNSUPPORTED"),
    (dict(max_batch=1 << 20, max_kv_len=1 << 30), "BIA_ERR_SHAPE"),   # > 2^31 states
])
def test_decode_graph_validation(change, status):
    args = dict(GRAPH, **change)
    if status is None:
        dg = bia.bia_decode_graph_create(**args)
        dg.close()
        return
    with pytest.raises(bia.BiaError) as e:
        bia.bia_decode_graph_create(**args)
    assert status in str(e.value)


def test_decode_graph_workspace_layout():
    """Flags, a fixed item per (request, kv head, partition), a merge per
    (request, kv head), then fp32 o and lse of every partial-state slot."""
    dg = bia.bia_decode_graph_create(**GRAPH)
    max_splits = 32768 // 2048
    items = 64 * 8 * max_splits
    states = items * 4
    def up(x):
        return (x + 255) // 256 * 256
    off_items = up(64 * 4)
    off_merges = up(off_items + items * 32)
    off_o = up(off_merges + 64 * 8 * 32)
    off_lse = up(off_o + states * 128 * 4)
    assert dg.workspace_bytes == up(off_lse + states * 4)
    dg.close()
    one = bia.bia_decode_graph_create(**dict(GRAPH, max_kv_len=2048))
    assert one.workspace_bytes < dg.workspace_bytes
    one.close()


def test_decode_graph_run_host_checks():
    """Checks that run before anything is enqueued (no GPU needed)."""
    lib = bia.load_library()
    dg = bia.bia_decode_graph_create(**GRAPH)
    h = ctypes.c_void_p(dg.handle)
    run = lib.bia_decode_graph_run
    nul = None
    assert run(None, 1, nul, nul, nul, nul, nul, 1.0, nul, nul, nul, 0, nul) != 0
    assert "NULL" in bia.bia_last_error()
    assert _lib._STATUS[run(h, 65, nul, nul, nul, nul, nul, 1.0, nul, nul, nul, 0, nul)] \
        == "BIA_ERR_SHAPE"
    assert _lib._STATUS[run(h, -1, nul, nul, nul, nul, nul, 1.0, nul, nul, nul, 0, nul)] \
        == "BIA_ERR_SHAPE"
    assert run(h, 0, nul, nul, nul, nul, nul, 1.0, nul, nul, nul, 0, nul) == 0   # no work
    assert _lib._STATUS[run(h, 0, nul, nul, nul, nul, nul, float("nan"), nul, nul, nul, 0,
                            nul)] == "BIA_ERR_INVALID_ARG"
    assert _lib._STATUS[run(h, 2, nul, nul, nul, nul, nul, 1.0, nul, nul, nul, 0, nul)] \
        == "BIA_ERR_INVALID_ARG"
    fake = ctypes.c_void_p(0x1000)
    assert _lib._STATUS[run(h, 2, fake, fake, fake, fake, fake, 1.0, fake, nul, fake, 16,
                            nul)] == "BIA_ERR_WORKSPACE"
    flags = np.zeros(1, dtype=np.int32)
    assert lib.bia_decode_graph_read_flags(None, fake, 1, _lib._ptr_i32(flags), nul) != 0
    assert lib.bia_decode_graph_read_flags(h, fake, 65, _lib._ptr_i32(flags), nul) != 0
    dg.close()
