"""Seeded synthetic inputs for paged causal attention.

This module builds inputs only. It holds none of the attention arithmetic and
is the one piece of code that both the CPU oracle checks and the GPU path see.

Layout of what it builds (the layout the library and the oracle both read):

* ``q``      bf16 ``[sum(qo_len), Hq, D]``, requests packed in order.
* ``k_pool`` / ``v_pool`` bf16 ``[num_pages, P, Hkv, D]`` (page, slot, kv head,
  dim), separate K and V pools.
* ``qo_indptr`` / ``kv_indptr`` int32 ``[B+1]``: cumulative query and KV token
  counts.
* ``page_table`` int32: request r's pages are
  ``page_table[page_off_r : page_off_r + ceil(kv_len_r / P)]`` with
  ``page_off_r = sum_{r' < r} ceil(kv_len_r' / P)``; token j of request r lives
  in page ``page_table[page_off_r + j // P]``, slot ``j % P``.

Values: every request draws its own K, V and Q from a generator seeded with
that request's own seed, in the order K, V, Q, as float32 N(0, 1) cast to
bf16 with round-to-nearest-even. A request therefore carries identical values
into any batch it joins, which is what batch-invariance tests need. Page ids
come from ``numpy.random.Generator(PCG64(batch_seed)).permutation(num_pages)``,
so the same request lands on different pages in different batches.

Pool memory that no request owns (unused pages, and slots past ``kv_len`` in a
request's last page) is filled with NaN, so a kernel that lets such memory into
a live product shows it in its output.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

PAGE_SIZE = 16

# Head shapes used by the workloads.
QWEN3_8B = dict(num_qo_heads=32, num_kv_heads=8, head_dim=128)
TINY = dict(num_qo_heads=4, num_kv_heads=1, head_dim=64)


@dataclass
class Request:
    """One request: ``qo_len`` new query tokens attending to ``kv_len`` keys.

    ``seed`` seeds this request's own value generator, so the request's q/k/v
    do not depend on the batch it is placed in.
    """

    qo_len: int
    kv_len: int
    seed: int


@dataclass
class PagedBatch:
    qo_indptr: np.ndarray  # int32 [B+1]
    kv_indptr: np.ndarray  # int32 [B+1]
    page_table: np.ndarray  # int32 [sum ceil(kv_len/P)]
    num_pages: int
    page_size: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    sm_scale: float
    q: torch.Tensor  # bf16 [sum qo, Hq, D]
    k_pool: torch.Tensor  # bf16 [num_pages, P, Hkv, D]
    v_pool: torch.Tensor  # bf16 [num_pages, P, Hkv, D]
    requests: List[Request] = field(default_factory=list)
    # Per-request contiguous copies (bf16, [kv_len, Hkv, D]) kept only when
    # asked for; small cases use them for a dense check that reads no page.
    k_seq: Optional[List[torch.Tensor]] = None
    v_seq: Optional[List[torch.Tensor]] = None

    @property
    def batch(self) -> int:
        return len(self.qo_indptr) - 1

    def qo_lens(self) -> np.ndarray:
        return np.diff(self.qo_indptr)

    def kv_lens(self) -> np.ndarray:
        return np.diff(self.kv_indptr)

    def pages_of(self, r: int) -> np.ndarray:
        """Page ids of request r, in token order."""
        counts = pages_needed(self.kv_lens(), self.page_size)
        off = int(counts[:r].sum())
        return self.page_table[off: off + int(counts[r])]

    def to(self, device) -> "PagedBatch":
        """Same batch with the tensors moved (index arrays stay on the host)."""
        return PagedBatch(
            self.qo_indptr, self.kv_indptr, self.page_table, self.num_pages,
            self.page_size, self.num_qo_heads, self.num_kv_heads, self.head_dim,
            self.sm_scale, self.q.to(device), self.k_pool.to(device),
            self.v_pool.to(device), list(self.requests), self.k_seq, self.v_seq)


def pages_needed(kv_lens: Sequence[int], page_size: int) -> np.ndarray:
    kv = np.asarray(kv_lens, dtype=np.int64)
    return (kv + page_size - 1) // page_size


def _normal_bf16(shape, gen: torch.Generator, device) -> torch.Tensor:
    return torch.randn(shape, generator=gen, dtype=torch.float32,
                       device=device).to(torch.bfloat16)


def draw_request(req: Request, num_qo_heads: int, num_kv_heads: int,
                 head_dim: int, device="cpu"):
    """K, V for ``kv_len`` tokens and Q for ``qo_len`` tokens, drawn in that
    order from a generator seeded with the request's seed."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(req.seed))
    k = _normal_bf16((req.kv_len, num_kv_heads, head_dim), gen, device)
    v = _normal_bf16((req.kv_len, num_kv_heads, head_dim), gen, device)
    q = _normal_bf16((req.qo_len, num_qo_heads, head_dim), gen, device)
    return k, v, q


def make_batch(requests: Sequence[Request], *, num_qo_heads: int,
               num_kv_heads: int, head_dim: int, num_pages: int, batch_seed: int,
               page_size: int = PAGE_SIZE, sm_scale: Optional[float] = None,
               device="cpu", keep_seq: bool = False,
               page_table: Optional[np.ndarray] = None) -> PagedBatch:
    """Build a paged batch from request specs (values drawn per request)."""
    reqs = list(requests)
    qs, ks, vs = [], [], []
    for r in reqs:
        k, v, q = draw_request(r, num_qo_heads, num_kv_heads, head_dim, device)
        qs.append(q)
        ks.append(k)
        vs.append(v)
    b = assemble_batch([r.qo_len for r in reqs], [r.kv_len for r in reqs], qs, ks,
                       vs, num_pages=num_pages, batch_seed=batch_seed,
                       page_size=page_size, sm_scale=sm_scale, device=device,
                       keep_seq=keep_seq, page_table=page_table)
    b.requests = reqs
    return b


def assemble_batch(qo_lens, kv_lens, q_list, k_list, v_list, *, num_pages: int,
                   batch_seed: int, page_size: int = PAGE_SIZE,
                   sm_scale: Optional[float] = None, device="cpu",
                   keep_seq: bool = False,
                   page_table: Optional[np.ndarray] = None) -> PagedBatch:
    """Place given per-request values into a paged pool.

    ``q_list[r] [qo_len, Hq, D]``, ``k_list[r]``/``v_list[r] [kv_len, Hkv, D]``
    (any float dtype; stored as bf16). Page ids are the first
    ``sum ceil(kv/P)`` entries of a PCG64 permutation of the pool unless
    ``page_table`` is given.
    """
    qo = np.asarray(qo_lens, dtype=np.int64)
    kv = np.asarray(kv_lens, dtype=np.int64)
    if np.any(qo > kv) or np.any(qo < 0):
        raise ValueError("each request needs 0 <= qo_len <= kv_len")
    num_kv_heads, head_dim = int(k_list[0].shape[1]), int(k_list[0].shape[2])
    num_qo_heads = int(q_list[0].shape[1])
    counts = pages_needed(kv, page_size)
    total_pages = int(counts.sum())
    if total_pages > num_pages:
        raise ValueError(f"pool of {num_pages} pages < {total_pages} needed")
    if page_table is None:
        rng = np.random.Generator(np.random.PCG64(batch_seed))
        page_table = rng.permutation(num_pages)[:total_pages].astype(np.int32)
    page_table = np.ascontiguousarray(page_table, dtype=np.int32)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(head_dim)

    qo_indptr = np.zeros(len(qo) + 1, dtype=np.int32)
    kv_indptr = np.zeros(len(kv) + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(qo)
    kv_indptr[1:] = np.cumsum(kv)

    pool_shape = (num_pages, page_size, num_kv_heads, head_dim)
    k_pool = torch.full(pool_shape, float("nan"), dtype=torch.bfloat16, device=device)
    v_pool = torch.full(pool_shape, float("nan"), dtype=torch.bfloat16, device=device)
    q = torch.empty((int(qo.sum()), num_qo_heads, head_dim), dtype=torch.bfloat16,
                    device=device)
    k_flat = k_pool.view(num_pages * page_size, num_kv_heads, head_dim)
    v_flat = v_pool.view(num_pages * page_size, num_kv_heads, head_dim)
    k_seq, v_seq = ([], []) if keep_seq else (None, None)
    off = 0
    for i in range(len(qo)):
        k = torch.as_tensor(k_list[i]).to(device=device, dtype=torch.bfloat16)
        v = torch.as_tensor(v_list[i]).to(device=device, dtype=torch.bfloat16)
        qr = torch.as_tensor(q_list[i]).to(device=device, dtype=torch.bfloat16)
        pages = torch.as_tensor(page_table[off: off + counts[i]].astype(np.int64),
                                device=device)
        j = torch.arange(int(kv[i]), device=device)
        slots = pages[j // page_size] * page_size + (j % page_size)
        k_flat[slots] = k
        v_flat[slots] = v
        q[qo_indptr[i]: qo_indptr[i + 1]] = qr
        if keep_seq:
            k_seq.append(k.cpu())
            v_seq.append(v.cpu())
        off += int(counts[i])
    return PagedBatch(qo_indptr, kv_indptr, page_table, num_pages, page_size,
                      num_qo_heads, num_kv_heads, head_dim, float(sm_scale), q,
                      k_pool, v_pool, [], k_seq, v_seq)


# Latent cache of multi-head latent attention (absorbed form): each token keeps
# one row of MLA_DK = 512 latent + 64 rope dims, shared by every q head; the
# values are its first MLA_DV dims.
MLA_DK = 576
MLA_DV = 512


def make_mla_batch(requests: Sequence[Request], *, num_qo_heads: int, num_pages: int,
                   batch_seed: int, sm_scale: Optional[float] = None, device="cpu",
                   keep_seq: bool = False,
                   page_table: Optional[np.ndarray] = None) -> PagedBatch:
    """Latent-cache batch: per request, ``kv_len`` latent rows ``[kv_len, 1,
    MLA_DK]`` and then ``qo_len`` queries ``[qo_len, Hq, MLA_DK]`` drawn from a
    generator seeded with the request's seed. ``k_pool`` is the latent pool
    ``[num_pages, 16, 1, MLA_DK]``; ``v_pool`` is a view of its first MLA_DV
    dims. The default scale is ``1 / sqrt(192)`` (the per-head q.k width of the
    un-absorbed form, 128 + 64)."""
    reqs = list(requests)
    kvs, qs = [], []
    for r in reqs:
        gen = torch.Generator(device=device)
        gen.manual_seed(int(r.seed))
        kvs.append(_normal_bf16((r.kv_len, 1, MLA_DK), gen, device))
        qs.append(_normal_bf16((r.qo_len, num_qo_heads, MLA_DK), gen, device))
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(192.0)
    b = assemble_batch([r.qo_len for r in reqs], [r.kv_len for r in reqs], qs, kvs, kvs,
                       num_pages=num_pages, batch_seed=batch_seed, sm_scale=sm_scale,
                       device=device, keep_seq=keep_seq, page_table=page_table)
    b.v_pool = b.k_pool[..., :MLA_DV]
    if keep_seq:
        b.v_seq = [k[..., :MLA_DV] for k in b.k_seq]
    b.requests = reqs
    return b


def rising_mla_batch(qo_lens, kv_lens, *, num_qo_heads: int, seed: int, num_pages: int,
                     rise: float = 3.0, device="cpu") -> PagedBatch:
    """Latent-cache batch whose logits climb along the sequence (the latent
    analogue of ``rising_batch``): latent row j of a request = (rise j /
    kv_len) + N(0, 0.25^2) per dim, q = 1 + N(0, 0.5^2), one PCG64 stream per
    request; about 0.19 base-2 units per key at kv_len 1000 with the default
    scale 1 / sqrt(192)."""
    kvs, qs = [], []
    for r, (qo, kv) in enumerate(zip(qo_lens, kv_lens)):
        g = np.random.Generator(np.random.PCG64(seed * 1013 + r))
        ramp = (rise * np.arange(kv, dtype=np.float32) / max(kv, 1))[:, None, None]
        kvs.append(torch.from_numpy(
            (ramp + 0.25 * g.standard_normal((kv, 1, MLA_DK), dtype=np.float32)).astype(np.float32)))
        qs.append(torch.from_numpy(
            (1.0 + 0.5 * g.standard_normal((qo, num_qo_heads, MLA_DK), dtype=np.float32))
            .astype(np.float32)))
    b = assemble_batch(qo_lens, kv_lens, qs, kvs, kvs, num_pages=num_pages, batch_seed=seed,
                       sm_scale=1.0 / math.sqrt(192.0), device=device)
    b.v_pool = b.k_pool[..., :MLA_DV]
    b.requests = [Request(qo, kv, seed * 1013 + r) for r, (qo, kv) in enumerate(zip(qo_lens, kv_lens))]
    return b


@dataclass
class Sequence1:
    """One long request stored once in a pool, viewed as chunked calls.

    ``q_full`` holds the query rows of all ``length`` tokens; a chunk
    ``[start, end)`` is the call with ``qo_len = end - start`` and
    ``kv_len = end`` on the same pages (prefix pages reused across chunks).
    """

    batch: PagedBatch  # the unchunked call: qo = kv = length
    length: int

    def chunk(self, start: int, end: int) -> PagedBatch:
        b = self.batch
        P = b.page_size
        pages = b.page_table[: (end + P - 1) // P]
        return PagedBatch(
            np.array([0, end - start], dtype=np.int32),
            np.array([0, end], dtype=np.int32),
            np.ascontiguousarray(pages), b.num_pages, P, b.num_qo_heads,
            b.num_kv_heads, b.head_dim, b.sm_scale, b.q[start:end], b.k_pool,
            b.v_pool, [Request(end - start, end, b.requests[0].seed)])


def make_sequence(length: int, *, seed: int, num_pages: int, device="cpu",
                  head=QWEN3_8B, page_size: int = PAGE_SIZE,
                  keep_seq: bool = False) -> Sequence1:
    b = make_batch([Request(length, length, seed)], num_pages=num_pages,
                   batch_seed=seed, page_size=page_size, device=device,
                   keep_seq=keep_seq, **head)
    return Sequence1(b, length)


def chunk_bounds(length: int, chunk: int):
    """[(start, end)] covering [0, length) in chunks of ``chunk`` tokens."""
    return [(s, min(s + chunk, length)) for s in range(0, length, chunk)]


# ---------------------------------------------------------------------------
# The workloads: the shapes and length mixes the attention is measured on.
# ---------------------------------------------------------------------------

def tiny_prefill(device="cpu", keep_seq=True) -> PagedBatch:
    """Two requests of 100 and 300 tokens, 4 q heads / 1 kv head, D = 64,
    26 of 64 pool pages, scale 1/sqrt(64)."""
    reqs = [Request(100, 100, 101), Request(300, 300, 102)]
    return make_batch(reqs, num_pages=64, batch_seed=1, device=device,
                      keep_seq=keep_seq, **TINY)


def tiny_sequence(device="cpu") -> Sequence1:
    """The 300-token request of the tiny workload on its own, for chunking
    (128 + 172 and other splits)."""
    b = make_batch([Request(300, 300, 102)], num_pages=64, batch_seed=1,
                   device=device, keep_seq=True, **TINY)
    return Sequence1(b, 300)


def rising_batch(qo_lens, kv_lens, *, num_qo_heads: int, num_kv_heads: int,
                 head_dim: int, seed: int, num_pages: int, rise: float = 6.0,
                 device="cpu") -> PagedBatch:
    """Keys whose logits climb along the sequence, so that a query's running
    max keeps rising by many base-2 units as its keys are visited.

    q = 1 + N(0, 0.5^2) per element, key j of a request = (rise j / kv_len) + N(0,
    0.25^2) per element, v ~ N(0, 1), all drawn from one PCG64 stream per
    request. With the 1/sqrt(D) scale a query's logit grows by about
    rise * D / sqrt(D) * log2(e) / kv_len base-2 units per key (about 0.1 at
    D = 128, kv_len 1000, rise 6)."""
    qs, ks, vs = [], [], []
    for r, (qo, kv) in enumerate(zip(qo_lens, kv_lens)):
        g = np.random.Generator(np.random.PCG64(seed * 1009 + r))
        ramp = (rise * np.arange(kv, dtype=np.float32) / max(kv, 1))[:, None, None]
        ks.append(torch.from_numpy(
            (ramp + 0.25 * g.standard_normal((kv, num_kv_heads, head_dim), dtype=np.float32))
            .astype(np.float32)))
        vs.append(torch.from_numpy(g.standard_normal((kv, num_kv_heads, head_dim),
                                                     dtype=np.float32)))
        qs.append(torch.from_numpy(
            (1.0 + 0.5 * g.standard_normal((qo, num_qo_heads, head_dim), dtype=np.float32))
            .astype(np.float32)))
    return assemble_batch(qo_lens, kv_lens, qs, ks, vs, num_pages=num_pages,
                          batch_seed=seed, device=device)


def qwen_prefill(device="cpu", batch=8, length=4096, num_pages=65536, seed=2):
    """Qwen3-8B-shaped layer prefill: ``batch`` requests of ``length`` tokens,
    32/8 heads, D = 128, pages permuted over a ``num_pages`` pool."""
    reqs = [Request(length, length, seed * 1000 + r) for r in range(batch)]
    return make_batch(reqs, num_pages=num_pages, batch_seed=seed, device=device,
                      **QWEN3_8B)


def decode_context_lengths(batch: int, seed: int = 4, max_ctx: int = 32768):
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(1, max_ctx + 1, size=batch)


def decode_batch(batch: int, *, seed: int = 4, num_pages: int = 131072,
                 device="cpu", probe: Optional[tuple] = None,
                 ctx_lens: Optional[Sequence[int]] = None,
                 head=QWEN3_8B, max_ctx: int = 32768) -> PagedBatch:
    """``batch`` decode requests (one query token each) with context lengths
    uniform in [1, max_ctx]. ``probe = (position, ctx, probe_seed)`` puts a
    request with its own seed at that position; page ids are re-drawn from
    ``seed`` so the probe moves to other pages whenever the batch changes."""
    if ctx_lens is None:
        ctx_lens = decode_context_lengths(batch, seed, max_ctx)
    reqs = [Request(1, int(c), seed * 100003 + r) for r, c in enumerate(ctx_lens)]
    if probe is not None:
        pos, pctx, pseed = probe
        reqs[pos] = Request(1, int(pctx), int(pseed))
    return make_batch(reqs, num_pages=num_pages, batch_seed=seed + 7919 * batch,
                      device=device, **head)


def mla_prefill(num_qo_heads: int, device="cpu", batch=4, length=4096, num_pages=16384,
                seed=12):
    """Latent-cache prefill: ``batch`` requests of ``length`` tokens, one
    576-dim cached head shared by ``num_qo_heads`` q heads."""
    reqs = [Request(length, length, seed * 1000 + r) for r in range(batch)]
    return make_mla_batch(reqs, num_qo_heads=num_qo_heads, num_pages=num_pages,
                          batch_seed=seed, device=device)


def mla_decode_batch(batch: int, num_qo_heads: int, *, seed: int = 4, num_pages: int = 131072,
                     device="cpu", max_ctx: int = 32768) -> PagedBatch:
    """``batch`` latent-cache decode requests with the context lengths of
    ``decode_batch`` (uniform in [1, max_ctx])."""
    ctx = decode_context_lengths(batch, seed, max_ctx)
    reqs = [Request(1, int(c), seed * 100003 + r) for r, c in enumerate(ctx)]
    return make_mla_batch(reqs, num_qo_heads=num_qo_heads, num_pages=num_pages,
                          batch_seed=seed + 7919 * batch, device=device)


def mixed_decode_lengths(n: int = 128, seed: int = 5, median: int = 4096,
                         sigma: float = 1.0, cap: int = 131072) -> np.ndarray:
    """Lognormal context lengths: round(exp(N(ln median, sigma^2))) in [1, cap]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = np.exp(rng.normal(math.log(median), sigma, size=n))
    return np.clip(np.round(x), 1, cap).astype(np.int64)


def host_subset(b: PagedBatch, reqs):
    """Host copies of the listed requests of a (device) batch: their q rows, a
    compact pool of just their pages (renumbered 0..n-1 in page-table order)
    and their indptrs. Renumbering pages does not change what attention
    computes. Returns (q, k_pool, v_pool, qo_indptr, kv_indptr, page_table,
    global_rows) where global_rows maps the copied q rows back to ``b.q``."""
    reqs = [int(r) for r in reqs]
    counts = pages_needed(b.kv_lens(), b.page_size)
    offs = np.concatenate([[0], np.cumsum(counts)])
    pages = (np.concatenate([b.page_table[offs[r]:offs[r + 1]] for r in reqs])
             if reqs else np.zeros(0, dtype=np.int32))
    idx = torch.as_tensor(pages.astype(np.int64), device=b.k_pool.device)
    kp = b.k_pool.index_select(0, idx).cpu()
    vp = b.v_pool.index_select(0, idx).cpu()
    qo = b.qo_lens()[reqs]
    kv = b.kv_lens()[reqs]
    qo_ip = np.concatenate([[0], np.cumsum(qo)]).astype(np.int64)
    kv_ip = np.concatenate([[0], np.cumsum(kv)]).astype(np.int64)
    rows = (np.concatenate([np.arange(b.qo_indptr[r], b.qo_indptr[r + 1]) for r in reqs])
            if reqs else np.zeros(0, dtype=np.int64))
    q = b.q[torch.as_tensor(rows, device=b.q.device)].cpu()
    return q, kp, vp, qo_ip, kv_ip, np.arange(len(pages)), rows


def jump_batch(qo_lens, kv_lens, jump_at, *, num_qo_heads: int, num_kv_heads: int,
               head_dim: int, seed: int, num_pages: int, c: float = 16.0,
               device="cpu") -> PagedBatch:
    """Keys whose logit leaps far above everything before it: per request and
    kv head a direction u ~ N(0, 1); q = u (of the head's kv head) + N(0,
    0.3^2); keys and values N(0, 1), except key ``jump_at[r]`` (if inside the
    request) = c u. With c = 16 that key scores about c |u|^2 / sqrt(D), some
    180 natural (260 base-2) units, far more than the 128 base-2 units past
    which exp2 against the row's earlier maximum overflows fp32. One PCG64
    stream per request."""
    qs, ks, vs = [], [], []
    g_size = num_qo_heads // num_kv_heads
    for r, (qo, kv) in enumerate(zip(qo_lens, kv_lens)):
        g = np.random.Generator(np.random.PCG64(seed * 1019 + r))
        u = g.standard_normal((num_kv_heads, head_dim), dtype=np.float32)
        k = g.standard_normal((kv, num_kv_heads, head_dim), dtype=np.float32)
        v = g.standard_normal((kv, num_kv_heads, head_dim), dtype=np.float32)
        j = int(jump_at[r])
        if 0 <= j < kv:
            k[j] = c * u
        uq = np.repeat(u, g_size, axis=0)[None]
        q = uq + 0.3 * g.standard_normal((qo, num_qo_heads, head_dim), dtype=np.float32)
        qs.append(torch.from_numpy(q))
        ks.append(torch.from_numpy(k))
        vs.append(torch.from_numpy(v))
    return assemble_batch(qo_lens, kv_lens, qs, ks, vs, num_pages=num_pages,
                          batch_seed=seed, device=device)


def identical_keys_batch(qo_lens, kv_lens, *, num_qo_heads: int, num_kv_heads: int,
                         head_dim: int, seed: int, num_pages: int,
                         device="cpu") -> PagedBatch:
    """Every key of a request (per kv head) is the same vector w ~ N(0, 1);
    q and v are N(0, 1). One PCG64 stream per request. Returned with the
    contiguous copies (``k_seq``/``v_seq``)."""
    qs, ks, vs = [], [], []
    for r, (qo, kv) in enumerate(zip(qo_lens, kv_lens)):
        g = np.random.Generator(np.random.PCG64(seed * 1021 + r))
        w = g.standard_normal((1, num_kv_heads, head_dim), dtype=np.float32)
        ks.append(torch.from_numpy(np.repeat(w, kv, axis=0)))
        vs.append(torch.from_numpy(g.standard_normal((kv, num_kv_heads, head_dim),
                                                     dtype=np.float32)))
        qs.append(torch.from_numpy(g.standard_normal((qo, num_qo_heads, head_dim),
                                                     dtype=np.float32)))
    return assemble_batch(qo_lens, kv_lens, qs, ks, vs, num_pages=num_pages,
                          batch_seed=seed, device=device, keep_seq=True)
