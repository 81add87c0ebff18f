"""Plain float64 causal attention over a paged KV cache (CPU oracle).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the CPU
baseline timing, never by the library.

Readings of the pages used here (they leave these points open):

* Causal alignment with a cached prefix is bottom-right: query i of a call with
  ``qo_len`` queries and ``kv_len`` keys sits at absolute position
  ``kv_len - qo_len + i`` and sees keys ``0..that position``. This is what makes
  a chunked prefill over cached prefix pages comparable with the unchunked one
  (sglang PR #43612, commit message and Summary).
* GQA groups are contiguous: q head h reads kv head ``h // (Hq / Hkv)``.
* ``lse`` is the natural-log log-sum-exp of the *scaled* logits.
* Pages: request r's token j is in page ``page_table[page_off_r + j // P]``,
  slot ``j % P``, with ``page_off_r = sum_{r' < r} ceil(kv_len_r' / P)``;
  pools are ``[num_pages, P, Hkv, D]``.
* Merge of partial states (split-KV, sglang PR #10417, Modifications): states
  with ``lse = -inf`` are empty and contribute nothing; the others combine as
  ``M = max lse_i``, ``w_i = exp(lse_i - M)``, ``o = sum w_i o_i / sum w_i``,
  ``lse = M + log sum w_i``.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np


def _f64(x) -> np.ndarray:
    """Host float64 copy of a numpy array or a (CPU or GPU) torch tensor."""
    if hasattr(x, "detach"):
        x = x.detach().float().cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def kv_head_of(h: int, group: int) -> int:
    """KV head read by q head ``h`` when ``group`` q heads share one kv head."""
    return h // group


def query_position(i: int, qo_len: int, kv_len: int) -> int:
    """Absolute KV position of the call's i-th query (bottom-right causal)."""
    return kv_len - qo_len + i


def page_offsets(kv_lens: Sequence[int], page_size: int) -> np.ndarray:
    """Index in the page table of each request's first page."""
    off = np.zeros(len(kv_lens), dtype=np.int64)
    total = 0
    for r, n in enumerate(kv_lens):
        off[r] = total
        total += -(-int(n) // page_size)  # ceil(n / P)
    return off


def _page_rows(pool, page: int, h_kv: int) -> np.ndarray:
    """float64 ``[P, D]``: every slot of one page for one kv head."""
    rows = pool[page, :, h_kv, :]
    if hasattr(rows, "detach"):
        rows = rows.detach().float().cpu().numpy()
    return np.asarray(rows, dtype=np.float64)


def gather_request_kv(pool, page_table, page_off: int, kv_len: int, h_kv: int):
    """Request's keys (or values) for one kv head, float64 ``[kv_len, D]``.

    Row j is ``pool[page_table[page_off + j // P], j % P, h_kv, :]``: the
    request's pages are read in page-table order and their slots in slot
    order, and rows past ``kv_len`` in the last page are dropped.
    """
    P = pool.shape[1]
    n_pages = -(-kv_len // P)
    parts = [_page_rows(pool, int(page_table[page_off + i]), h_kv)
             for i in range(n_pages)]
    if not parts:
        return np.zeros((0, pool.shape[3]), dtype=np.float64)
    return np.concatenate(parts, axis=0)[:kv_len]


def attend(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray,
           positions: np.ndarray, sm_scale: float):
    """Softmax attention of each query row over keys ``0..position``.

    ``q_rows [n, D]``, ``K, V [kv_len, D]``, ``positions [n]``. For row i:
    ``s_j = sm_scale * q_i . k_j`` for ``j <= positions[i]``;
    ``lse_i = m + ln sum_j exp(s_j - m)`` with ``m = max_j s_j``;
    ``out_i = sum_j exp(s_j - lse_i) v_j``.
    """
    S = sm_scale * (q_rows @ K.T)
    j = np.arange(K.shape[0])[None, :]
    S = np.where(j <= positions[:, None], S, -np.inf)
    m = S.max(axis=1)
    lse = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
    out = np.exp(S - lse[:, None]) @ V
    return out, lse


def attention_paged(q, k_pool, v_pool, qo_indptr, kv_indptr, page_table,
                    num_kv_heads: int, sm_scale: float,
                    rows: Optional[Sequence[int]] = None,
                    row_block: int = 1024):
    """Causal attention of every (or of the selected) query rows of a batch.

    ``q [sum qo, Hq, Dk]``; ``k_pool [num_pages, P, Hkv, Dk]``, ``v_pool
    [num_pages, P, Hkv, Dv]``; indptrs ``[B+1]``. ``rows`` selects global
    query rows (indices into ``q``'s first axis); rows not selected are left
    NaN. Returns ``out [sum qo, Hq, Dv]`` and ``lse [sum qo, Hq]`` in float64.
    """
    qo_indptr = np.asarray(qo_indptr, dtype=np.int64)
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    page_table = np.asarray(page_table, dtype=np.int64)
    q = _f64(q)
    n_q, Hq, _ = q.shape
    D = v_pool.shape[3]          # output width: the value dim (may differ from q's)
    group = Hq // num_kv_heads
    P = k_pool.shape[1]
    B = len(qo_indptr) - 1
    qo_lens = np.diff(qo_indptr)
    kv_lens = np.diff(kv_indptr)
    offs = page_offsets(kv_lens, P)
    want = None if rows is None else np.zeros(n_q, dtype=bool)
    if want is not None:
        want[np.asarray(rows, dtype=np.int64)] = True

    out = np.full((n_q, Hq, D), np.nan)
    lse = np.full((n_q, Hq), np.nan)
    for r in range(B):
        qo_len, kv_len = int(qo_lens[r]), int(kv_lens[r])
        local = np.arange(qo_len)
        if want is not None:
            local = local[want[qo_indptr[r] + local]]
        if local.size == 0:
            continue
        for h_kv in range(num_kv_heads):
            K = gather_request_kv(k_pool, page_table, offs[r], kv_len, h_kv)
            V = gather_request_kv(v_pool, page_table, offs[r], kv_len, h_kv)
            for h in range(Hq):
                if kv_head_of(h, group) != h_kv:
                    continue
                for b0 in range(0, local.size, row_block):
                    ii = local[b0: b0 + row_block]
                    pos = np.array([query_position(int(i), qo_len, kv_len) for i in ii])
                    o, s = attend(q[qo_indptr[r] + ii, h, :], K, V, pos, sm_scale)
                    out[qo_indptr[r] + ii, h, :] = o
                    lse[qo_indptr[r] + ii, h] = s
    return out, lse


def decode_paged(q, k_pool, v_pool, kv_indptr, page_table, num_kv_heads: int,
                 sm_scale: float, requests: Optional[Sequence[int]] = None):
    """Decode: one query token per request, seeing all ``kv_len`` keys.

    ``q [B, Hq, D]``. This is ``attention_paged`` with ``qo_len = 1``.
    """
    B = len(kv_indptr) - 1
    qo_indptr = np.arange(B + 1)
    return attention_paged(q, k_pool, v_pool, qo_indptr, kv_indptr, page_table,
                           num_kv_heads, sm_scale, rows=requests)


def merge_states(v, s, state_indptr):
    """Merge partial attention states row by row.

    ``v [n_states, H, D]`` partial outputs, ``s [n_states, H]`` their
    natural-log lse (``-inf`` = empty state), ``state_indptr [n_rows+1]``: row
    i merges states ``state_indptr[i] .. state_indptr[i+1]-1``. A row whose
    states are all empty gives ``o = 0``, ``lse = -inf``.
    """
    v = _f64(v)
    s = _f64(s)
    indptr = np.asarray(state_indptr, dtype=np.int64)
    n_rows = len(indptr) - 1
    H, D = v.shape[1], v.shape[2]
    out = np.zeros((n_rows, H, D))
    lse = np.full((n_rows, H), -np.inf)
    for i in range(n_rows):
        lo, hi = indptr[i], indptr[i + 1]
        for h in range(H):
            si = s[lo:hi, h]
            live = si != -np.inf
            if not live.any():
                continue
            M = si[live].max()
            w = np.exp(si[live] - M)
            out[i, h] = (w[:, None] * v[lo:hi, h][live]).sum(axis=0) / w.sum()
            lse[i, h] = M + math.log(w.sum())
    return out, lse


def latent_values(kv_pool, v_dim: int):
    """Values of latent (absorbed multi-head latent) attention: the first
    ``v_dim`` dims of every cached latent row (the rest is the rope part,
    which only enters the scores)."""
    return kv_pool[..., :v_dim]


def mla_attention_paged(q, kv_pool, qo_indptr, kv_indptr, page_table, sm_scale: float,
                        v_dim: int, rows: Optional[Sequence[int]] = None):
    """Causal attention over a paged latent cache: every q head scores against
    the full latent row (``Dk`` dims: latent + rope) of one shared cache head
    and averages its first ``v_dim`` dims. The pages name this MLA wrapper as
    the one path without a deterministic mode (sglang PR #43612, commit
    message and Summary); the reading here is the absorbed form, with the
    same causal alignment and page layout as the other calls.

    ``q [sum qo, Hq, Dk]``; ``kv_pool [num_pages, P, Dk]`` or
    ``[num_pages, P, 1, Dk]``. Returns ``out [sum qo, Hq, v_dim]`` and
    ``lse [sum qo, Hq]`` (float64).
    """
    k_pool = kv_pool if kv_pool.ndim == 4 else kv_pool[:, :, None, :]
    return attention_paged(q, k_pool, latent_values(k_pool, v_dim), qo_indptr, kv_indptr,
                           page_table, 1, sm_scale, rows=rows)
