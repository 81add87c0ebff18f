"""Latent (MLA) attention on the GPU: parity with the float64 oracle, and the
same invariances as the other calls (a request's bits do not depend on the
batch around it, on on-grid chunking, or on prefill vs decode for its last
token)."""
import numpy as np
import pytest
import torch

import invariant_paged_kv_amd as bia
import oracle
import workloads as W
from gpu_util import LSE_TOL, OUT_TOL, bits_equal, page_table_dev, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def kv_view(b: W.PagedBatch):
    """The latent pool as the library takes it: [num_pages, 16, 576]."""
    return b.k_pool.view(b.num_pages, b.page_size, W.MLA_DK)


def run_mla(b: W.PagedBatch, mode=bia.BIA_MODE_PREFILL, split=None):
    if split is None:
        split = bia.BIA_PREFILL_SPLIT if mode == bia.BIA_MODE_PREFILL else bia.BIA_DECODE_SPLIT
    plan = bia.bia_plan_create(mode, b.qo_indptr, b.kv_indptr, b.page_table,
                               num_qo_heads=b.num_qo_heads, num_kv_heads=1,
                               head_dim=W.MLA_DK, num_pages=b.num_pages, split_size=split,
                               flags=bia.BIA_PLAN_MLA)
    n = b.q.shape[0]
    out = torch.full((n, b.num_qo_heads, W.MLA_DV), float("nan"), dtype=torch.bfloat16,
                     device=DEV)
    lse = torch.full((n, b.num_qo_heads), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=DEV)
    fn = bia.bia_mla_prefill_paged if mode == bia.BIA_MODE_PREFILL else bia.bia_mla_decode_paged
    fn(plan, b.q, kv_view(b), page_table_dev(b), b.sm_scale, out, lse, ws)
    torch.cuda.synchronize()
    plan.close()
    return out, lse


def mla_parity(b: W.PagedBatch, out, lse, what, local_rows=None):
    reqs = [r for r in range(b.batch) if b.qo_lens()[r] > 0]
    q, kp, _, qo_ip, kv_ip, pt, grows = W.host_subset(b, reqs)
    sel = None
    if local_rows is not None:
        sel = np.concatenate([qo_ip[i] + np.asarray(local_rows[r], dtype=np.int64)
                              for i, r in enumerate(reqs)])
    o_ref, l_ref = oracle.mla_attention_paged(q, kp, qo_ip, kv_ip, pt, b.sm_scale, W.MLA_DV,
                                              rows=sel)
    if sel is None:
        sel = np.arange(len(grows))
    idx = torch.as_tensor(grows[sel], device=DEV)
    e_out = float(np.max(np.abs(out[idx].double().cpu().numpy() - o_ref[sel])))
    e_lse = float(np.max(np.abs(lse[idx].double().cpu().numpy() - l_ref[sel])))
    say(f"{what}: rows={len(sel)} max|out err|={e_out:.3e} max|lse err|={e_lse:.3e}")
    assert np.isfinite(e_out) and e_out <= OUT_TOL, f"{what}: out error {e_out}"
    assert np.isfinite(e_lse) and e_lse <= LSE_TOL, f"{what}: lse error {e_lse}"


@pytest.mark.parametrize("hq", [16, 128])
@pytest.mark.parametrize("split", [256, 4096])
def test_mla_prefill_parity(hq, split):
    """Ragged lengths (not multiples of the 32-key tile or of the q tile), a
    request with no new tokens, one whose chunk starts mid-sequence, and a
    split that makes rows span several partitions (merged in fixed order)."""
    if hq == 16:
        reqs = [W.Request(300, 700, 901), W.Request(0, 40, 902), W.Request(101, 101, 903),
                W.Request(1, 333, 904)]
    else:
        reqs = [W.Request(150, 530, 911), W.Request(37, 37, 912), W.Request(2, 17, 913)]
    say(f"mla prefill parity hq={hq} split={split}")
    b = W.make_mla_batch(reqs, num_qo_heads=hq, num_pages=256, batch_seed=41, device=DEV)
    out, lse = run_mla(b, split=split)
    mla_parity(b, out, lse, f"mla prefill hq={hq} split={split}")


@pytest.mark.parametrize("hq", [16, 32, 64, 128])
def test_mla_decode_parity(hq):
    """One query token per request; lengths around and past the 2048-key
    decode split. 16 heads take the one-wave-per-item kernel; 32 and 64 the
    128-row kernel with two and four of its eight waves holding rows."""
    kv = [1, 17, 2048, 2049, 5000]
    reqs = [W.Request(1, c, 920 + i) for i, c in enumerate(kv)]
    say(f"mla decode parity hq={hq}")
    b = W.make_mla_batch(reqs, num_qo_heads=hq, num_pages=1024, batch_seed=43, device=DEV)
    out, lse = run_mla(b, mode=bia.BIA_MODE_DECODE)
    mla_parity(b, out, lse, f"mla decode hq={hq}")


@pytest.mark.parametrize("split", [8192, 16384])
def test_mla_large_splits(split):
    """Splits above 2048 up to the largest allowed (16384): 16-head decode
    then runs the 128-row kernel instead of the one-wave-per-item one, and
    the prefill items of a 64-token chunk over a 12000-token prefix loop over
    up to 375 32-key tiles, with rows spanning one or two partitions."""
    kv = [1, 2049, 9000, 17000]
    reqs = [W.Request(1, c, 960 + i) for i, c in enumerate(kv)]
    say(f"mla decode hq=16 split={split}")
    b = W.make_mla_batch(reqs, num_qo_heads=16, num_pages=2048, batch_seed=47, device=DEV)
    out, lse = run_mla(b, mode=bia.BIA_MODE_DECODE, split=split)
    mla_parity(b, out, lse, f"mla decode hq=16 split={split}")
    reqs = [W.Request(64, 12000, 965), W.Request(64, 64, 966)]
    say(f"mla prefill hq=16 split={split}")
    b = W.make_mla_batch(reqs, num_qo_heads=16, num_pages=1024, batch_seed=48, device=DEV)
    out, lse = run_mla(b, split=split)
    mla_parity(b, out, lse, f"mla prefill hq=16 split={split}")


@pytest.mark.parametrize("hq", [8, 64])
def test_mla_prefill_parity_tile_tokens(hq):
    """128-row tiles hold 128 / min(Hq, 128) tokens: 16 at 8 heads, 2 at 64.
    Token counts that are not multiples of that (a request's last tile
    partly empty), a one-token request and a chunk starting mid-sequence."""
    reqs = [W.Request(37, 300, 951), W.Request(1, 1, 952), W.Request(17, 17, 953),
            W.Request(5, 129, 954)]
    say(f"mla prefill tile tokens hq={hq}")
    b = W.make_mla_batch(reqs, num_qo_heads=hq, num_pages=128, batch_seed=75, device=DEV)
    out, lse = run_mla(b, split=256)
    mla_parity(b, out, lse, f"mla prefill hq={hq} split=256")


def test_mla_many_partitions_hq32():
    """32 q heads (four tokens per 128-row tile) at split 64: rows span up to
    ten partitions, merged in fixed order at 512 dims; ragged lengths."""
    reqs = [W.Request(67, 600, 981), W.Request(3, 64, 982), W.Request(1, 65, 983),
            W.Request(130, 130, 984)]
    say("mla hq=32 split=64")
    b = W.make_mla_batch(reqs, num_qo_heads=32, num_pages=128, batch_seed=71, device=DEV)
    out, lse = run_mla(b, split=64)
    mla_parity(b, out, lse, "mla prefill hq=32 split=64")


def test_mla_decode_hq8():
    """8 q heads: half of one wave's rows are heads, the rest and three waves
    are idle rows."""
    reqs = [W.Request(1, c, 990 + i) for i, c in enumerate([1, 31, 32, 33, 2047, 4100])]
    say("mla decode hq=8")
    b = W.make_mla_batch(reqs, num_qo_heads=8, num_pages=512, batch_seed=73, device=DEV)
    out, lse = run_mla(b, mode=bia.BIA_MODE_DECODE)
    mla_parity(b, out, lse, "mla decode hq=8")


@pytest.mark.parametrize("hq", [8, 64])
def test_mla_one_key_is_the_value(hq):
    """A row that sees one key returns that key's first 512 dims exactly (its
    weight is exactly 1)."""
    say(f"mla one key hq={hq}")
    b = W.make_mla_batch([W.Request(1, 1, 931), W.Request(5, 5, 932)], num_qo_heads=hq,
                         num_pages=16, batch_seed=3, device=DEV, keep_seq=True)
    out, _ = run_mla(b)
    for r, row in [(0, 0), (1, 1)]:
        v0 = b.k_seq[r][0, 0, :W.MLA_DV].to(DEV)
        for h in range(hq):
            assert bits_equal(out[row, h], v0), (r, h)


@pytest.mark.parametrize("hq", [16, 128])
def test_mla_batch_invariance(hq):
    """A request's out and lse bits are the same alone and inside batches of
    other sizes and compositions (other pages, other positions)."""
    target = W.Request(200, 900, 941)
    others = [W.Request(64, 64, 942), W.Request(3, 2500, 943), W.Request(0, 10, 944),
              W.Request(129, 300, 945)]
    say(f"mla batch invariance hq={hq}")
    res = []
    for k, reqs in enumerate([[target], [others[0], target], others + [target],
                              [others[1], target, others[3]]]):
        b = W.make_mla_batch(reqs, num_qo_heads=hq, num_pages=512, batch_seed=50 + k,
                             device=DEV)
        out, lse = run_mla(b, split=256)
        i = reqs.index(target)
        r0, r1 = int(b.qo_indptr[i]), int(b.qo_indptr[i + 1])
        res.append((out[r0:r1].clone(), lse[r0:r1].clone()))
    for o, l in res[1:]:
        assert bits_equal(o, res[0][0]) and bits_equal(l, res[0][1])


def test_mla_chunk_invariance():
    """Chunks that start on the 128-token grid reproduce the unchunked call
    bit for bit, at a split that cuts partitions inside the sequence."""
    hq, L = 16, 1000
    say("mla chunk invariance")
    b = W.make_mla_batch([W.Request(L, L, 951)], num_qo_heads=hq, num_pages=128,
                         batch_seed=9, device=DEV)
    full_o, full_l = run_mla(b, split=256)
    for cuts in [[0, 256, 512, 1000], [0, 128, 384, 896, 1000]]:
        for s, e in zip(cuts[:-1], cuts[1:]):
            pages = b.page_table[: (e + 15) // 16]
            cb = W.PagedBatch(np.array([0, e - s], np.int32), np.array([0, e], np.int32),
                              np.ascontiguousarray(pages), b.num_pages, 16, hq, 1, W.MLA_DK,
                              b.sm_scale, b.q[s:e].contiguous(), b.k_pool, b.v_pool,
                              [W.Request(e - s, e, 951)])
            o, l = run_mla(cb, split=256)
            assert bits_equal(o, full_o[s:e]) and bits_equal(l, full_l[s:e]), (s, e)


def test_mla_decode_batch_invariance_hq16():
    """Decode with 16 q heads (one wave per request): a probe request's bits
    are the same alone and at other positions in batches of other sizes,
    with other pages."""
    probe = W.Request(1, 5000, 999)
    say("mla decode batch invariance hq=16")
    ref = None
    for k, n in enumerate([1, 3, 8, 13]):
        others = [W.Request(1, 1 + (977 * i + 131 * k) % 9000, 1000 + 37 * k + i)
                  for i in range(n - 1)]
        pos = (5 * k) % n
        reqs = others[:pos] + [probe] + others[pos:]
        b = W.make_mla_batch(reqs, num_qo_heads=16, num_pages=4096, batch_seed=80 + k,
                             device=DEV)
        out, lse = run_mla(b, mode=bia.BIA_MODE_DECODE)
        o, l = out[pos].clone(), lse[pos].clone()
        if ref is None:
            ref = (o, l)
            mla_parity(b, out, lse, "mla decode hq=16 probe")
        else:
            assert bits_equal(o, ref[0]) and bits_equal(l, ref[1]), n


@pytest.mark.parametrize("hq", [32, 64, 128])
def test_mla_decode_equals_prefill_last_row(hq):
    """With 32 or more q heads, decode runs the prefill kernel on a one-token
    tile, so it equals the last row of the request's prefill at the same
    split bit for bit (the row's arithmetic does not depend on its tile).
    With 16 or fewer heads decode takes 16-key tiles of its own and is only
    held to parity and batch invariance."""
    kv = [100, 2048, 3001]
    say(f"mla decode vs prefill hq={hq}")
    full = W.make_mla_batch([W.Request(c, c, 960 + i) for i, c in enumerate(kv)],
                            num_qo_heads=hq, num_pages=512, batch_seed=61, device=DEV)
    po, pl = run_mla(full, split=2048)
    last = full.qo_indptr[1:] - 1
    dec = W.PagedBatch(np.arange(len(kv) + 1, dtype=np.int32), full.kv_indptr,
                       full.page_table, full.num_pages, 16, hq, 1, W.MLA_DK, full.sm_scale,
                       full.q[torch.as_tensor(last, device=DEV)].contiguous(), full.k_pool,
                       full.v_pool, [])
    do, dl = run_mla(dec, mode=bia.BIA_MODE_DECODE, split=2048)
    idx = torch.as_tensor(last, device=DEV)
    assert bits_equal(do, po[idx].contiguous()) and bits_equal(dl, pl[idx].contiguous())


def test_mla_rejects_wrong_shapes():
    b = W.make_mla_batch([W.Request(4, 20, 970)], num_qo_heads=16, num_pages=8,
                         batch_seed=1, device=DEV)
    plan = bia.bia_plan_create(bia.BIA_MODE_PREFILL, b.qo_indptr, b.kv_indptr, b.page_table,
                               num_qo_heads=16, num_kv_heads=1, head_dim=W.MLA_DK,
                               num_pages=b.num_pages, split_size=4096, flags=bia.BIA_PLAN_MLA)
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=DEV)
    out = torch.empty(4, 16, W.MLA_DK, dtype=torch.bfloat16, device=DEV)   # 576, not 512
    lse = torch.empty(4, 16, dtype=torch.float32, device=DEV)
    with pytest.raises(bia.BiaError):
        bia.bia_mla_prefill_paged(plan, b.q, kv_view(b), page_table_dev(b), b.sm_scale, out,
                                  lse, ws)
    with pytest.raises(bia.BiaError):
        bia.bia_prefill_paged(plan, b.q, b.k_pool, b.k_pool, page_table_dev(b), b.sm_scale,
                              out, lse, ws)
    plan.close()


@pytest.mark.parametrize("hq", [16, 128])
def test_mla_rising_logits(hq):
    """Latent logits that climb along the sequence: rows raise their running
    max mid-row again and again; the 1500-key request spans partitions whose
    states merge with very different lse. Decode covers the one-wave kernel
    (16 heads) and the 128-row kernel (128 heads)."""
    say(f"mla rising logits hq={hq}")
    b = W.rising_mla_batch([400, 200, 9], [400, 1500, 9], num_qo_heads=hq, seed=91,
                           num_pages=256, rise=1.5, device=DEV)
    out, lse = run_mla(b, split=256)
    mla_parity(b, out, lse, f"mla rising prefill hq={hq}")
    ctx = [1, 300, 2048, 2049, 4000]
    d = W.rising_mla_batch([1] * len(ctx), ctx, num_qo_heads=hq, seed=92, num_pages=1024,
                           rise=1.5, device=DEV)
    out, lse = run_mla(d, mode=bia.BIA_MODE_DECODE)
    mla_parity(d, out, lse, f"mla rising decode hq={hq}")
