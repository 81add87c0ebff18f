"""Benchmark: Qwen3-8B-shaped paged attention on one MI355X.

One step is one pass of the whole path over one batch of synthetic inputs
already resident in HBM: plan (host) + causal paged prefill of 8 requests x
4096 tokens (32 q / 8 kv heads, D 128, page 16, pages permuted over a 64K-page
pool, split 4096) + paged decode of 64 requests with contexts uniform in
[1, 32768] (split 2048, partial states merged in fixed order).

Prints ONE JSON line. ``value`` is prefill attention TFLOP/s (algorithmic
FLOPs 4 * D * Hq * sum over rows of visible keys, divided by the prefill
call's time from HIP events on its stream); ``decode.value`` is decode KV
GB/s (bytes of K and V read once per kv head, plus q, out, lse and page ids).
``roofline`` is the prefill kernel against the bf16 MFMA peak,
``decode.roofline`` the decode kernel against HBM bandwidth. ``cpu_baseline``
is the float64 CPU oracle timed on the same inputs (the whole prefill and the
whole decode batch), with the host's CPU model and core counts. ``mixed`` is
the long-context workload: a 65536-token prefill in four 16384-token chunks,
each step beside 128 lognormal-context decodes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill attn TFLOP/s + decode KV GB/s (Qwen3-8B shape), % roofline, bit-invariant"
MFMA_BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 4096 flop/clk x 2.4 GHz, dense
HBM_PEAK_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "invariant_paged_kv_amd", "csrc", "bia.hip")
COUNTERS = os.path.join(ROOT, "profiles", "hbm_traffic__qwen3_8b_prefill_8x4096_decode_b64.txt")


def prefill_flops(qo_lens, kv_lens, num_qo_heads, head_dim) -> float:
    """4 * D * Hq * sum over query rows of the keys each row sees (QK^T and
    PV over visible keys only)."""
    total = 0
    for qo, kv in zip(qo_lens, kv_lens):
        qo, kv = int(qo), int(kv)
        first = kv - qo + 1            # keys seen by the first query row
        total += qo * (first + kv) // 2
    return 4.0 * head_dim * num_qo_heads * total


def decode_bytes(kv_lens, num_qo_heads, num_kv_heads, head_dim, page_size=16) -> float:
    kv = np.asarray(kv_lens, dtype=np.int64)
    b = kv.sum() * num_kv_heads * head_dim * 2 * 2            # K and V, bf16
    b += len(kv) * num_qo_heads * head_dim * 2 * 2            # q in, out
    b += len(kv) * num_qo_heads * 4                           # lse
    b += 4 * ((kv + page_size - 1) // page_size).sum()         # page ids
    return float(b)


def source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None if absent or taken on other kernel source."""
    if not os.path.exists(COUNTERS):
        return None
    text = open(COUNTERS).read()
    m = re.search(r"source_sha256_16:\s*(\w+)", text)
    if not m or m.group(1) != source_hash():
        return None
    m = re.search(rf"^{kernel}_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    return float(m.group(1)) if m else None


class Timer:
    """HIP events on the stream the library launches on."""

    def __init__(self, torch, stream):
        self.torch = torch
        self.stream = stream
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        return e

    def stop(self, s):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        self.pairs.append((s, e))

    def mean_ms(self):
        return float(np.mean([s.elapsed_time(e) for s, e in self.pairs]))


def _oracle_threads() -> int:
    """Threads of the BLAS pool the float64 oracle's matrix products run on."""
    from threadpoolctl import threadpool_info
    return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))


def host_info() -> dict:
    """The host the oracle is timed on: CPU model, CPUs this process may run
    on, BLAS threads the oracle uses."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "host_cpus_available": len(os.sched_getaffinity(0)),
            "blas_threads": _oracle_threads()}


def cpu_baseline_prefill(b, n=8):
    """The float64 CPU oracle on the first ``n`` requests of the prefill batch
    (4096 tokens each, all 32 q heads; n = 8 is the whole workload), same
    inputs."""
    import oracle
    import workloads as W
    q, kp, vp, qo_ip, kv_ip, pt, _ = W.host_subset(b, list(range(n)))
    t = time.perf_counter()
    oracle.attention_paged(q, kp, vp, qo_ip, kv_ip, pt, b.num_kv_heads, b.sm_scale)
    dt = time.perf_counter() - t
    fl = prefill_flops(np.diff(qo_ip), np.diff(kv_ip), b.num_qo_heads, b.head_dim)
    what = "the whole prefill workload" if n == b.batch else f"{n}/{b.batch} of the prefill workload"
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": _oracle_threads(), "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"prefill requests 0..{n - 1} of {b.batch} (4096 tokens each, all 32 q "
                      f"heads): {what}, same seeded inputs", **host_info()}


def cpu_baseline_decode(b, n=64):
    """The float64 CPU oracle on the first ``n`` decode requests (n = 64 is
    the whole batch)."""
    import oracle
    import workloads as W
    reqs = list(range(n))
    q, kp, vp, qo_ip, kv_ip, pt, _ = W.host_subset(b, reqs)
    t = time.perf_counter()
    oracle.decode_paged(q, kp, vp, kv_ip, pt, b.num_kv_heads, b.sm_scale)
    dt = time.perf_counter() - t
    by = decode_bytes(np.diff(kv_ip), b.num_qo_heads, b.num_kv_heads, b.head_dim)
    return {"value": round(by / dt / 1e9, 4), "unit": "GB/s",
            "cores": _oracle_threads(), "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"decode requests 0..{n - 1} of {b.batch} "
                      f"({int(np.diff(kv_ip).sum())} context tokens), same seeded inputs",
            **host_info()}


def mixed_steps(torch, bia, W, stream, dev, rounds=3):
    """The mixed long-context workload: one 65536-token request prefilled in
    four 16384-token chunks (chunk c: qo 16384, kv 16384 (c + 1), over its
    cached prefix pages, split 4096) plus 128 decodes with lognormal contexts
    (median 4096, sigma 1, cap 131072; split 2048). One step = prefill chunk c
    + the 128 decodes. Per step: prefill TFLOP/s and decode GB/s from HIP
    events on the stream, with their roofline fractions; averaged over
    ``rounds`` passes of the four steps after one untimed pass."""
    seq = W.make_sequence(65536, seed=5, num_pages=8192, device=dev)
    ctx = W.mixed_decode_lengths()
    db = W.decode_batch(128, ctx_lens=ctx, seed=5, num_pages=131072, device=dev,
                        max_ctx=131072)
    heads = dict(num_qo_heads=32, num_kv_heads=8, head_dim=128)
    chunks = [seq.chunk(lo, hi) for lo, hi in W.chunk_bounds(65536, 16384)]
    s_pt = torch.as_tensor(seq.batch.page_table, dtype=torch.int32, device=dev)
    d_pt = torch.as_tensor(db.page_table, dtype=torch.int32, device=dev)
    p_out = torch.empty(16384, 32, 128, dtype=torch.bfloat16, device=dev)
    p_lse = torch.empty(16384, 32, dtype=torch.float32, device=dev)
    d_out = torch.empty_like(db.q)
    d_lse = torch.empty(db.q.shape[:2], dtype=torch.float32, device=dev)

    def plans(ch):
        pp = bia.bia_plan_create(bia.BIA_MODE_PREFILL, ch.qo_indptr, ch.kv_indptr,
                                 ch.page_table, num_pages=ch.num_pages,
                                 split_size=bia.BIA_PREFILL_SPLIT, **heads)
        dp = bia.bia_plan_create(bia.BIA_MODE_DECODE, db.qo_indptr, db.kv_indptr,
                                 db.page_table, num_pages=db.num_pages,
                                 split_size=bia.BIA_DECODE_SPLIT, **heads)
        return pp, dp

    p_bytes, d_bytes_ws = 256, 256
    for ch in chunks:
        pp, dp = plans(ch)
        p_bytes = max(p_bytes, pp.workspace_bytes)
        d_bytes_ws = max(d_bytes_ws, dp.workspace_bytes)
        pp.close(), dp.close()
    p_ws = torch.empty(p_bytes, dtype=torch.uint8, device=dev)
    d_ws = torch.empty(d_bytes_ws, dtype=torch.uint8, device=dev)
    timers = [(Timer(torch, stream), Timer(torch, stream)) for _ in chunks]
    for r in range(rounds + 1):
        for c, ch in enumerate(chunks):
            pp, dp = plans(ch)
            pt_t, dt_t = timers[c]
            s = pt_t.start() if r else None
            bia.bia_prefill_paged(pp, ch.q, ch.k_pool, ch.v_pool, s_pt, ch.sm_scale, p_out,
                                  p_lse, p_ws, stream)
            if r:
                pt_t.stop(s)
                s = dt_t.start()
            bia.bia_decode_paged(dp, db.q, db.k_pool, db.v_pool, d_pt, db.sm_scale, d_out,
                                 d_lse, d_ws, stream)
            if r:
                dt_t.stop(s)
            pp.close(), dp.close()
    torch.cuda.synchronize()
    d_bytes = decode_bytes(db.kv_lens(), 32, 8, 128)
    steps = []
    for c, ch in enumerate(chunks):
        p_ms, d_ms = timers[c][0].mean_ms(), timers[c][1].mean_ms()
        fl = prefill_flops(ch.qo_lens(), ch.kv_lens(), 32, 128)
        tf = fl / (p_ms * 1e-3) / 1e12
        gbs = d_bytes / (d_ms * 1e-3) / 1e9
        steps.append({"chunk": [16384 * c, 16384 * (c + 1)], "prefill_ms": round(p_ms, 4),
                      "prefill_TFLOP/s": round(tf, 1),
                      "prefill_frac_mfma": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                      "decode_ms": round(d_ms, 4), "decode_GB/s": round(gbs, 1),
                      "decode_frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                      "step_ms": round(p_ms + d_ms, 4)})
    tot_fl = sum(prefill_flops(ch.qo_lens(), ch.kv_lens(), 32, 128) for ch in chunks)
    tot_p = sum(x["prefill_ms"] for x in steps)
    tot_d = sum(x["decode_ms"] for x in steps)
    del seq, db, chunks, p_ws, d_ws
    return {"workload": "65536-token prefill in 4 chunks of 16384 + 128 decodes, lognormal "
                        "contexts (median 4096, sigma 1, cap 131072)",
            "decode_kv_tokens": int(ctx.sum()), "steps": steps,
            "prefill_TFLOP/s": round(tot_fl / (tot_p * 1e-3) / 1e12, 1),
            "decode_GB/s": round(4 * d_bytes / (tot_d * 1e-3) / 1e9, 1),
            "ms_per_step": round((tot_p + tot_d) / 4, 4)}


def copy_bandwidth(torch, stream, dev, gib=2, reps=10):
    """Device-to-device copy of a ``gib`` GiB buffer: (read + write bytes) /
    mean time, GB/s. The achievable-HBM reference the decode is compared to."""
    n = gib << 29                                   # int16 elements
    src = torch.ones(n, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    t = Timer(torch, stream)
    for _ in range(reps):
        s = t.start()
        dst.copy_(src)
        t.stop(s)
    torch.cuda.synchronize()
    ms = t.mean_ms()
    del src, dst
    return 2.0 * (n * 2) / (ms * 1e-3) / 1e9


def decode_sweep(torch, bia, W, db, d_pt, stream, dev, sizes=(1, 8, 16, 32, 64), reps=20):
    """Planned decode of the first B requests of the B = 64 batch (same pool),
    with a 512 MB scratch buffer read between calls so small batches are not
    served from the 256 MB last-level cache. A read, not a write: written
    scratch lines stay dirty in that cache and are written back while the
    next call runs, which cost short calls up to 45 % (B = 2) in measurement.
    GB/s and ms per call."""
    scratch = torch.ones(1 << 29, dtype=torch.uint8, device=dev)
    rows = []
    for B in sizes:
        kv = db.kv_indptr[: B + 1]
        n_pages = int(((np.diff(kv) + 15) // 16).sum())
        sub = W.PagedBatch(db.qo_indptr[: B + 1], kv, db.page_table[:n_pages], db.num_pages,
                           db.page_size, db.num_qo_heads, db.num_kv_heads, db.head_dim,
                           db.sm_scale, db.q[:B].contiguous(), db.k_pool, db.v_pool)
        plan = bia.bia_plan_create(bia.BIA_MODE_DECODE, sub.qo_indptr, sub.kv_indptr,
                                   sub.page_table, num_pages=sub.num_pages,
                                   split_size=bia.BIA_DECODE_SPLIT, num_qo_heads=32,
                                   num_kv_heads=8, head_dim=128)
        ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=dev)
        out = torch.empty_like(sub.q)
        lse = torch.empty(sub.q.shape[:2], dtype=torch.float32, device=dev)
        t = Timer(torch, stream)
        for i in range(reps + 2):
            scratch.sum()
            s = t.start()
            bia.bia_decode_paged(plan, sub.q, sub.k_pool, sub.v_pool, d_pt, sub.sm_scale,
                                 out, lse, ws, stream)
            t.stop(s)
        torch.cuda.synchronize()
        t.pairs = t.pairs[2:]
        ms = t.mean_ms()
        by = decode_bytes(sub.kv_lens(), 32, 8, 128)
        rows.append({"batch": B, "kv_tokens": int(sub.kv_lens().sum()), "ms": round(ms, 4),
                     "GB/s": round(by / (ms * 1e-3) / 1e9, 1)})
        plan.close()
    del scratch
    return rows


def decode_graph_replay(torch, bia, db, d_pt, stream, dev, ref_out, ref_lse, reps=20):
    """The graph-capturable decode of the B = 64 batch, captured once in a HIP
    graph and replayed: ms per replay, GB/s, and whether its bits equal the
    planned decode's. Replays and planned calls (one plan, made once) are
    timed alternately on one stream, so both see the same GPU state: the
    clocks and caches change over the first few dozen calls after a pause."""
    B = db.batch
    dg = bia.bia_decode_graph_create(max_batch=B, num_qo_heads=32, num_kv_heads=8,
                                     head_dim=128, num_pages=db.num_pages,
                                     max_kv_len=32768, page_table_capacity=int(d_pt.numel()))
    ind = torch.as_tensor(db.kv_indptr, dtype=torch.int32, device=dev)
    out = torch.empty_like(db.q)
    lse = torch.empty(db.q.shape[:2], dtype=torch.float32, device=dev)
    ws = torch.empty(dg.workspace_bytes, dtype=torch.uint8, device=dev)

    def call():
        bia.bia_decode_graph_run(dg, B, ind, db.q, db.k_pool, db.v_pool, d_pt, db.sm_scale,
                                 out, lse, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    out.zero_()
    g.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(out.view(torch.int16), ref_out.view(torch.int16)) and
                torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)))
    plan = bia.bia_plan_create(bia.BIA_MODE_DECODE, db.qo_indptr, db.kv_indptr,
                               db.page_table, num_pages=db.num_pages,
                               split_size=bia.BIA_DECODE_SPLIT, num_qo_heads=32,
                               num_kv_heads=8, head_dim=128)
    p_out = torch.empty_like(db.q)
    p_lse = torch.empty_like(lse)
    pws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=dev)
    cur = torch.cuda.current_stream(dev)
    tg, tp = Timer(torch, cur), Timer(torch, cur)
    for i in range(reps + 2):
        s = tg.start()
        g.replay()
        tg.stop(s)
        s = tp.start()
        bia.bia_decode_paged(plan, db.q, db.k_pool, db.v_pool, d_pt, db.sm_scale, p_out, p_lse,
                             pws, cur)
        tp.stop(s)
    torch.cuda.synchronize()
    tg.pairs, tp.pairs = tg.pairs[2:], tp.pairs[2:]
    ms, planned_ms = tg.mean_ms(), tp.mean_ms()
    plan.close()
    by = decode_bytes(db.kv_lens(), 32, 8, 128)
    del g
    dg.close()
    return {"ms": round(ms, 4), "GB/s": round(by / (ms * 1e-3) / 1e9, 1),
            "bit_equal_to_planned": same, "planned_alternating_ms": round(planned_ms, 4)}


def mla_flops(qo_lens, kv_lens, num_qo_heads) -> float:
    """2 * (576 + 512) * Hq per (query row, visible key): scores over the
    576-dim latent + rope row, values over its first 512 dims."""
    total = 0
    for qo, kv in zip(qo_lens, kv_lens):
        qo, kv = int(qo), int(kv)
        total += qo * ((kv - qo + 1) + kv) // 2
    return 2.0 * (576 + 512) * num_qo_heads * total


def mla_bytes(kv_lens, num_qo_heads, page_size=16) -> float:
    """Cached latent rows read once, q in, out and lse out, page ids."""
    kv = np.asarray(kv_lens, dtype=np.int64)
    b = kv.sum() * 576 * 2
    b += len(kv) * num_qo_heads * (576 * 2 + 512 * 2 + 4)
    b += 4 * ((kv + page_size - 1) // page_size).sum()
    return float(b)


def mla_extra(torch, bia, W, stream, dev, reps=10):
    """Latent (MLA) attention: causal prefill of 4 x 4096 tokens and decode of
    64 requests with contexts U[1, 32768], at 16 and 128 q heads (one GPU's
    heads of a 128-head model under 8-way head parallelism, and all of them).
    Prefill against the bf16 MFMA peak; decode against HBM bandwidth (bytes
    of the cached rows read once) and, for 128 heads, also as TFLOP/s."""
    res = {}
    for hq in (16, 128):
        row = {}
        for mode in ("prefill", "decode"):
            if mode == "prefill":
                b = W.mla_prefill(hq, device=dev)
                m, split = bia.BIA_MODE_PREFILL, bia.BIA_PREFILL_SPLIT
                fn = bia.bia_mla_prefill_paged
            else:
                b = W.mla_decode_batch(64, hq, device=dev)
                m, split = bia.BIA_MODE_DECODE, bia.BIA_DECODE_SPLIT
                fn = bia.bia_mla_decode_paged
            pt = torch.as_tensor(b.page_table, dtype=torch.int32, device=dev)
            kv = b.k_pool.view(b.num_pages, 16, 576)
            out = torch.empty(b.q.shape[0], hq, 512, dtype=torch.bfloat16, device=dev)
            lse = torch.empty(b.q.shape[0], hq, dtype=torch.float32, device=dev)
            plan = bia.bia_plan_create(m, b.qo_indptr, b.kv_indptr, b.page_table,
                                       num_qo_heads=hq, num_kv_heads=1, head_dim=576,
                                       num_pages=b.num_pages, split_size=split,
                                       flags=bia.BIA_PLAN_MLA)
            ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=dev)
            t = Timer(torch, stream)
            for i in range(reps + 2):
                s = t.start()
                fn(plan, b.q, kv, pt, b.sm_scale, out, lse, ws, stream)
                t.stop(s)
            torch.cuda.synchronize()
            t.pairs = t.pairs[2:]
            ms = t.mean_ms()
            fl = mla_flops(b.qo_lens(), b.kv_lens(), hq)
            tf = fl / (ms * 1e-3) / 1e12
            e = {"ms": round(ms, 4), "TFLOP/s": round(tf, 1),
                 "frac_mfma": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
            if mode == "decode":
                gbs = mla_bytes(b.kv_lens(), hq) / (ms * 1e-3) / 1e9
                e["GB/s"] = round(gbs, 1)
                e["frac_hbm"] = round(gbs / HBM_PEAK_GBS, 4)
            row[mode] = e
            plan.close()
            del b, kv, out, lse, ws, pt
        res[f"hq{hq}"] = row
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the decode batch sweep, the graph-replay decode and the "
                         "copy-bandwidth reference")
    ap.add_argument("--mla-only", action="store_true",
                    help="time only the latent (MLA) calls and print their numbers")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first copy a 1 GiB buffer 3 times, so a counter run also "
                         "records a plain copy of known size (HBM-byte calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the library runs on one "
              "GPU and this benchmark measures that GPU's share of the attention at its "
              "real shape; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import invariant_paged_kv_amd as bia
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bia.load_library()
    stream = torch.cuda.current_stream(dev)
    if args.calibrate_copy:
        src = torch.ones(1 << 29, dtype=torch.int16, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.mla_only:
        print(json.dumps({"mla": mla_extra(torch, bia, W, stream, dev)}), flush=True)
        return

    pb = W.qwen_prefill(device=dev)                       # 8 x 4096, 64K-page pool
    db = W.decode_batch(64, seed=4, num_pages=131072, device=dev)
    p_pt = torch.as_tensor(pb.page_table, dtype=torch.int32, device=dev)
    d_pt = torch.as_tensor(db.page_table, dtype=torch.int32, device=dev)
    p_out = torch.empty_like(pb.q)
    p_lse = torch.empty(pb.q.shape[:2], dtype=torch.float32, device=dev)
    d_out = torch.empty_like(db.q)
    d_lse = torch.empty(db.q.shape[:2], dtype=torch.float32, device=dev)
    heads = dict(num_qo_heads=32, num_kv_heads=8, head_dim=128)

    plan_s = {"prefill": [], "decode": []}

    def make_plans(timed=False):
        t0 = time.perf_counter()
        pp = bia.bia_plan_create(bia.BIA_MODE_PREFILL, pb.qo_indptr, pb.kv_indptr,
                                 pb.page_table, num_pages=pb.num_pages,
                                 split_size=bia.BIA_PREFILL_SPLIT, **heads)
        t1 = time.perf_counter()
        dp = bia.bia_plan_create(bia.BIA_MODE_DECODE, db.qo_indptr, db.kv_indptr,
                                 db.page_table, num_pages=db.num_pages,
                                 split_size=bia.BIA_DECODE_SPLIT, **heads)
        t2 = time.perf_counter()
        if timed:
            plan_s["prefill"].append(t1 - t0)
            plan_s["decode"].append(t2 - t1)
        return pp, dp

    pp, dp = make_plans()
    p_ws = torch.empty(max(pp.workspace_bytes, 256), dtype=torch.uint8, device=dev)
    d_ws = torch.empty(max(dp.workspace_bytes, 256), dtype=torch.uint8, device=dev)
    pp.close()
    dp.close()

    p_timer, d_timer = Timer(torch, stream), Timer(torch, stream)

    def step(timed: bool):
        pp, dp = make_plans(timed)                 # a1: plan from the lengths alone
        s = p_timer.start() if timed else None
        bia.bia_prefill_paged(pp, pb.q, pb.k_pool, pb.v_pool, p_pt, pb.sm_scale, p_out,
                              p_lse, p_ws, stream)
        if timed:
            p_timer.stop(s)
            s = d_timer.start()
        bia.bia_decode_paged(dp, db.q, db.k_pool, db.v_pool, d_pt, db.sm_scale, d_out,
                             d_lse, d_ws, stream)
        if timed:
            d_timer.stop(s)
        # destroyed while their work is still queued: the pinned work-list
        # blocks go back to the library's pool, no device wait
        pp.close()
        dp.close()

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    ref_p = p_out.clone()
    ref_d = d_out.clone()

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    invariant = bool(torch.equal(ref_p.view(torch.int16), p_out.view(torch.int16)) and
                     torch.equal(ref_d.view(torch.int16), d_out.view(torch.int16)))
    extras = {}
    if not args.no_extras:
        extras["copy_gbs"] = copy_bandwidth(torch, stream, dev)
        extras["sweep"] = decode_sweep(torch, bia, W, db, d_pt, stream, dev)
        extras["graph"] = decode_graph_replay(torch, bia, db, d_pt, stream, dev, d_out, d_lse)
        extras["mla"] = mla_extra(torch, bia, W, stream, dev)
        extras["mixed"] = mixed_steps(torch, bia, W, stream, dev)

    p_flops = prefill_flops(pb.qo_lens(), pb.kv_lens(), 32, 128)
    d_bytes = decode_bytes(db.kv_lens(), 32, 8, 128)
    p_ms = p_timer.mean_ms()
    d_ms = d_timer.mean_ms()
    p_tflops = p_flops / (p_ms * 1e-3) / 1e12
    d_gbs = d_bytes / (d_ms * 1e-3) / 1e9

    p_traffic = read_traffic("prefill")
    d_traffic = read_traffic("decode")
    result = {
        "metric": METRIC,
        "value": round(p_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "Qwen3-8B-shaped attention layer: causal paged prefill 8 x 4096 "
                        "tokens + paged decode of 64 requests, contexts U[1, 32768]",
            "num_qo_heads": 32, "num_kv_heads": 8, "head_dim": 128, "page_size": 16,
            "prefill": {"requests": 8, "tokens": 4096, "pool_pages": pb.num_pages,
                        "split": bia.BIA_PREFILL_SPLIT},
            "decode": {"requests": 64, "ctx": "uniform [1, 32768]",
                       "total_kv_tokens": int(db.kv_lens().sum()),
                       "pool_pages": db.num_pages, "split": bia.BIA_DECODE_SPLIT},
        },
        "prefill_ms": round(p_ms, 4),
        "roofline": {
            "bound": "mfma", "achieved": round(p_tflops, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(p_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": p_traffic,
        },
        "decode": {
            "value": round(d_gbs, 1), "unit": "GB/s", "ms": round(d_ms, 4),
            "roofline": {
                "bound": "hbm", "achieved": round(d_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(d_gbs / HBM_PEAK_GBS, 4),
                "traffic": d_traffic,
            },
        },
        "bit_invariant_across_steps": invariant,
        "plan_ms": {
            "prefill": round(float(np.median(plan_s["prefill"])) * 1e3, 4),
            "decode": round(float(np.median(plan_s["decode"])) * 1e3, 4),
            "what": "host time of bia_plan_create (median over the timed steps), "
                    "included in ms_per_step, not in the GPU call timings"},
    }
    if extras:
        copy = extras["copy_gbs"]
        result["copy_bandwidth"] = {
            "value": round(copy, 1), "unit": "GB/s",
            "what": "2 GiB device-to-device copy, (read + write bytes) / time"}
        result["decode"]["frac_of_copy"] = round(d_gbs / copy, 4)
        result["decode"]["sweep"] = extras["sweep"]
        result["decode"]["graph_replay"] = extras["graph"]
        result["mla"] = extras["mla"]
        result["mixed"] = extras["mixed"]
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_prefill(pb)
        result["decode"]["cpu_baseline"] = cpu_baseline_decode(db)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
