"""Helpers for the GPU tests: run the library on a PagedBatch, and compute
the CPU oracle on host copies of the same inputs (only the pages the chosen
requests own are copied to the host)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import invariant_paged_kv_amd as bia
import oracle
import workloads as W

OUT_TOL = 2e-2   # max abs error on bf16 outputs vs the float64 oracle
LSE_TOL = 1e-3   # max abs error on fp32 lse


def say(*a):
    """Name the case before a GPU step, flushed, so a fault names it."""
    print("[gpu]", *a, file=sys.stderr, flush=True)


def device():
    return torch.device("cuda:0")


def page_table_dev(b: W.PagedBatch):
    pt = b.page_table if b.page_table.size else np.zeros(1, dtype=np.int32)
    return torch.as_tensor(pt, dtype=torch.int32, device=b.q.device)


def run_prefill(b: W.PagedBatch, split=bia.BIA_PREFILL_SPLIT, want_lse=True):
    plan = bia.bia_plan_create(bia.BIA_MODE_PREFILL, b.qo_indptr, b.kv_indptr,
                               b.page_table, num_qo_heads=b.num_qo_heads,
                               num_kv_heads=b.num_kv_heads, head_dim=b.head_dim,
                               num_pages=b.num_pages, split_size=split)
    dev = b.q.device
    out = torch.full_like(b.q, float("nan"))
    lse = torch.full(b.q.shape[:2], float("nan"), dtype=torch.float32, device=dev) \
        if want_lse else None
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=dev)
    bia.bia_prefill_paged(plan, b.q, b.k_pool, b.v_pool, page_table_dev(b), b.sm_scale,
                          out, lse, ws)
    torch.cuda.synchronize()
    plan.close()
    return out, lse


def run_decode(b: W.PagedBatch, split=bia.BIA_DECODE_SPLIT):
    plan = bia.bia_plan_create(bia.BIA_MODE_DECODE, b.qo_indptr, b.kv_indptr,
                               b.page_table, num_qo_heads=b.num_qo_heads,
                               num_kv_heads=b.num_kv_heads, head_dim=b.head_dim,
                               num_pages=b.num_pages, split_size=split)
    dev = b.q.device
    out = torch.full_like(b.q, float("nan"))
    lse = torch.full(b.q.shape[:2], float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=dev)
    bia.bia_decode_paged(plan, b.q, b.k_pool, b.v_pool, page_table_dev(b), b.sm_scale,
                         out, lse, ws)
    torch.cuda.synchronize()
    plan.close()
    return out, lse


def sample_rows(qo_len: int, edge=128, every=61):
    """Rows of one request the oracle checks on large cases: the first and
    last ``edge`` query tokens and every ``every``-th one."""
    r = set(range(min(edge, qo_len))) | set(range(max(0, qo_len - edge), qo_len))
    r |= set(range(0, qo_len, every))
    return np.array(sorted(r), dtype=np.int64)


def oracle_for(b: W.PagedBatch, reqs, local_rows=None):
    """float64 oracle for the listed requests. ``local_rows`` maps request ->
    rows (within the request) to compute; None = all. Returns
    (global_rows, out [n, Hq, D], lse [n, Hq])."""
    q, kp, vp, qo_ip, kv_ip, pt, grows = W.host_subset(b, reqs)
    sel = None
    if local_rows is not None:
        sel = np.concatenate([qo_ip[i] + np.asarray(local_rows[r], dtype=np.int64)
                              for i, r in enumerate(reqs)])
    out, lse = oracle.attention_paged(q, kp, vp, qo_ip, kv_ip, pt, b.num_kv_heads,
                                      b.sm_scale, rows=sel)
    if sel is None:
        sel = np.arange(len(grows))
    return grows[sel], out[sel], lse[sel]


def parity(out_gpu, lse_gpu, rows, out_ref, lse_ref):
    """(max abs error of out, of lse) over the given global rows."""
    idx = torch.as_tensor(rows, device=out_gpu.device)
    og = out_gpu[idx].double().cpu().numpy()
    e_out = float(np.max(np.abs(og - out_ref))) if og.size else 0.0
    e_lse = 0.0
    if lse_gpu is not None:
        lg = lse_gpu[idx].double().cpu().numpy()
        e_lse = float(np.max(np.abs(lg - lse_ref))) if lg.size else 0.0
    return e_out, e_lse


def assert_parity(out_gpu, lse_gpu, b, reqs=None, local_rows=None, what=""):
    if reqs is None:
        reqs = [r for r in range(b.batch) if b.qo_lens()[r] > 0]
    rows, o_ref, l_ref = oracle_for(b, reqs, local_rows)
    e_out, e_lse = parity(out_gpu, lse_gpu, rows, o_ref, l_ref)
    say(f"{what}: rows={len(rows)} max|out err|={e_out:.3e} max|lse err|={e_lse:.3e}")
    assert np.isfinite(e_out) and e_out <= OUT_TOL, f"{what}: out error {e_out}"
    assert np.isfinite(e_lse) and e_lse <= LSE_TOL, f"{what}: lse error {e_lse}"
    return e_out, e_lse


def bits_equal(a, b) -> bool:
    """Bitwise equality of two tensors (NaN payloads and signed zeros count)."""
    if a.shape != b.shape or a.dtype != b.dtype:
        return False
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)
