"""KV append on the GPU: writing each request's new tokens into its pages
reproduces the generator's pool bit for bit and touches nothing else; read
back through the oracle's own page/slot gather, every request's keys and
values equal the generator's never-paged rows; and a prefill over the
appended pool equals the prefill over the original pool and meets oracle
parity."""
import numpy as np
import pytest
import torch

import invariant_paged_kv_amd as bia
import oracle
import workloads as W
from gpu_util import assert_parity, bits_equal, page_table_dev, run_prefill, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def new_token_slots(b: W.PagedBatch):
    """Flat pool slot of every new token, in q-row order."""
    P = b.page_size
    counts = W.pages_needed(b.kv_lens(), P)
    offs = np.concatenate([[0], np.cumsum(counts)])
    slots = []
    for r in range(b.batch):
        qo, kv = int(b.qo_lens()[r]), int(b.kv_lens()[r])
        pages = b.page_table[offs[r]:offs[r + 1]].astype(np.int64)
        for j in range(kv - qo, kv):
            slots.append(pages[j // P] * P + j % P)
    return np.array(slots, dtype=np.int64)


@pytest.mark.parametrize("mode", ["prefill", "decode"])
def test_append_then_attend(mode):
    say(f"append ({mode})")
    if mode == "prefill":
        reqs = [W.Request(77, 300, 701), W.Request(0, 20, 702), W.Request(129, 129, 703),
                W.Request(1, 1000, 704), W.Request(40, 41, 705)]
    else:
        reqs = [W.Request(1, int(c), 710 + i) for i, c in enumerate([1, 17, 2048, 5000])]
    b = W.make_batch(reqs, num_pages=1024, batch_seed=31, device=DEV, keep_seq=True,
                     **W.QWEN3_8B)
    slots = torch.as_tensor(new_token_slots(b), device=DEV)
    Hkv, D = b.num_kv_heads, b.head_dim
    # the new tokens' rows, from the generator's never-paged copies
    k_new = torch.cat([b.k_seq[r][int(b.kv_lens()[r] - b.qo_lens()[r]):]
                       for r in range(b.batch)]).to(DEV).contiguous()
    v_new = torch.cat([b.v_seq[r][int(b.kv_lens()[r] - b.qo_lens()[r]):]
                       for r in range(b.batch)]).to(DEV).contiguous()
    k_pool = b.k_pool.clone()
    v_pool = b.v_pool.clone()
    k_pool.view(-1, Hkv, D)[slots] = float("nan")      # the new tokens' slots are stale
    v_pool.view(-1, Hkv, D)[slots] = float("nan")
    m = bia.BIA_MODE_PREFILL if mode == "prefill" else bia.BIA_MODE_DECODE
    split = bia.BIA_PREFILL_SPLIT if mode == "prefill" else bia.BIA_DECODE_SPLIT
    plan = bia.bia_plan_create(m, b.qo_indptr, b.kv_indptr, b.page_table, num_pages=b.num_pages,
                               split_size=split, **W.QWEN3_8B)
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=DEV)
    bia.bia_append_paged_kv(plan, k_new, v_new, page_table_dev(b), k_pool, v_pool, ws)
    torch.cuda.synchronize()
    plan.close()
    # bitwise: NaN payloads in untouched slots compare equal as bits
    assert bits_equal(k_pool, b.k_pool) and bits_equal(v_pool, b.v_pool)
    # the oracle's gather (its page/slot mapping) over the appended pool gives
    # back every request's rows, old and new, exactly
    offs = oracle.page_offsets(b.kv_lens(), b.page_size)
    kp_h, vp_h = k_pool.cpu(), v_pool.cpu()
    for r in range(b.batch):
        kv = int(b.kv_lens()[r])
        for h in range(Hkv):
            kg = oracle.gather_request_kv(kp_h, b.page_table, int(offs[r]), kv, h)
            vg = oracle.gather_request_kv(vp_h, b.page_table, int(offs[r]), kv, h)
            assert np.array_equal(kg, b.k_seq[r][:, h, :].double().numpy())
            assert np.array_equal(vg, b.v_seq[r][:, h, :].double().numpy())
    if mode == "prefill":
        o1, l1 = run_prefill(b)
        b2 = W.PagedBatch(b.qo_indptr, b.kv_indptr, b.page_table, b.num_pages, b.page_size,
                          b.num_qo_heads, b.num_kv_heads, b.head_dim, b.sm_scale, b.q,
                          k_pool, v_pool)
        o2, l2 = run_prefill(b2)
        assert bits_equal(o1, o2) and bits_equal(l1, l2)
        assert_parity(o2, l2, b2, what="prefill over the appended pool")
