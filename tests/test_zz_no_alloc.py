"""bia_decode_paged_static (workspace in the library's static device array,
no allocation) against bia_decode_paged (caller's workspace): the same bits,
on two calls in a row, the second with a smaller batch; and a plan whose
workspace exceeds the static array is rejected before anything runs."""
import numpy as np
import pytest
import torch

import invariant_paged_kv_amd as bia
import workloads as W
from gpu_util import bits_equal, page_table_dev, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _plan(b):
    return bia.bia_plan_create(bia.BIA_MODE_DECODE, b.qo_indptr, b.kv_indptr, b.page_table,
                               num_qo_heads=b.num_qo_heads, num_kv_heads=b.num_kv_heads,
                               head_dim=b.head_dim, num_pages=b.num_pages,
                               split_size=bia.BIA_DECODE_SPLIT)


def test_static_workspace_matches_caller_workspace():
    big = W.decode_batch(24, seed=31, num_pages=32768, device=DEV, max_ctx=20000)
    small = W.decode_batch(5, ctx_lens=[1, 2049, 300, 4096, 17], seed=32, num_pages=4096,
                           device=DEV)
    runs = []
    for name, b in (("B=24", big), ("B=5", small)):
        p = _plan(b)
        assert 0 < p.workspace_bytes <= bia.BIA_STATIC_WORKSPACE_BYTES
        assert p.num_states > 0, "the case should merge partitions"
        pt = page_table_dev(b)
        ws = torch.empty(p.workspace_bytes, dtype=torch.uint8, device=DEV)
        ref = torch.full_like(b.q, float("nan"))
        ref_lse = torch.full(b.q.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
        say(f"static workspace: bia_decode_paged {name}")
        bia.bia_decode_paged(p, b.q, b.k_pool, b.v_pool, pt, b.sm_scale, ref, ref_lse, ws)
        torch.cuda.synchronize()
        runs.append((name, b, p, pt, ref, ref_lse))
    outs = []
    for name, b, p, pt, _, _ in runs:   # two calls in a row, the second smaller
        out = torch.full_like(b.q, float("nan"))
        lse = torch.full(b.q.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
        say(f"static workspace: bia_decode_paged_static {name}")
        bia.bia_decode_paged_static(p, b.q, b.k_pool, b.v_pool, pt, b.sm_scale, out, lse)
        outs.append((out, lse))
    torch.cuda.synchronize()
    for (name, b, p, pt, ref, ref_lse), (out, lse) in zip(runs, outs):
        assert bits_equal(out, ref), f"{name}: out differs from bia_decode_paged"
        assert bits_equal(lse, ref_lse), f"{name}: lse differs from bia_decode_paged"
        p.close()


def test_static_workspace_rejects_large_plans():
    """64 requests of 131072 keys need ~70 MB of partial states: rejected with
    BIA_ERR_WORKSPACE before any launch (pages repeat over a small pool)."""
    B, ctx, pool = 64, 131072, 1024
    qo = np.arange(B + 1, dtype=np.int32)
    kv = (np.arange(B + 1, dtype=np.int64) * ctx).astype(np.int32)
    pt = (np.arange(B * ctx // 16) % pool).astype(np.int32)
    p = bia.bia_plan_create(bia.BIA_MODE_DECODE, qo, kv, pt, num_pages=pool,
                            split_size=bia.BIA_DECODE_SPLIT, **W.QWEN3_8B)
    assert p.workspace_bytes > bia.BIA_STATIC_WORKSPACE_BYTES
    q = torch.zeros(B, 32, 128, dtype=torch.bfloat16, device=DEV)
    kp = torch.zeros(pool, 16, 8, 128, dtype=torch.bfloat16, device=DEV)
    out = torch.zeros_like(q)
    lse = torch.zeros(B, 32, dtype=torch.float32, device=DEV)
    say("static workspace: oversized plan is rejected")
    with pytest.raises(bia.BiaError) as e:
        bia.bia_decode_paged_static(p, q, kp, kp, torch.as_tensor(pt, device=DEV), 0.1,
                                    out, lse)
    assert str(e.value).startswith("BIA_ERR_WORKSPACE")
    assert "static workspace" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    p.close()
