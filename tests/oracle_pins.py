"""Checks that pin the CPU oracle to facts outside itself.

Each ``pin_*`` raises ``AssertionError`` when the oracle disagrees with:

* a closed form (one visible key; identical keys),
* the hand-worked 3-token causal example in ``golden/three_token_causal.txt``,
* a dense library computation (``torch.nn.functional.scaled_dot_product_attention``
  and ``torch.logsumexp`` in float64) over the generator's contiguous,
  never-paged copies of K and V,
* exact invariances (chunked rows equal unchunked rows; decode equals the last
  prefill row; relocating pages changes nothing; V + c gives out + c; GQA
  equals MHA with repeated kv heads),
* for latent (MLA) attention: one key, identical keys, and a dense library
  computation over the contiguous latent rows.

The pins reach the oracle through the module ``oracle.attention`` so that
``test_oracle_mutations.py`` can swap one of its functions for a copy with a
planted mistake and show that some pin fails.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

import oracle.attention as A
import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))
TOL = 1e-12


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite oracle values"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol * max(1.0, np.max(np.abs(b)) if b.size else 1.0), \
        f"{what}: max abs diff {err:.3e}"


def _run(b: W.PagedBatch, rows=None):
    return A.attention_paged(b.q, b.k_pool, b.v_pool, b.qo_indptr, b.kv_indptr,
                             b.page_table, b.num_kv_heads, b.sm_scale, rows=rows)


def _f64(t):
    return t.detach().double().cpu().numpy()


# --------------------------------------------------------------------- pins --

def pin_one_key():
    """kv_len = 1: out = v_0 and lse = s_0 = sm_scale * q . k_0, for a decode
    request and for row 0 of a fresh prefill; GQA with 2 kv heads."""
    reqs = [W.Request(1, 1, 11), W.Request(3, 3, 12)]
    b = W.make_batch(reqs, num_qo_heads=4, num_kv_heads=2, head_dim=64,
                     num_pages=8, batch_seed=3, keep_seq=True)
    out, lse = _run(b)
    for r, row in ((0, 0), (1, 1)):
        q = _f64(b.q[row])                     # [Hq, D]
        k0 = _f64(b.k_seq[r][0])               # [Hkv, D]
        v0 = _f64(b.v_seq[r][0])
        for h in range(4):
            hk = h // 2
            _close(out[row, h], v0[hk], 0.0, "one key: out = v0")
            _close(lse[row, h], b.sm_scale * float(q[h] @ k0[hk]), TOL,
                   "one key: lse = s0")


def pin_identical_keys():
    """All keys of a kv head equal: row at position p gets
    out = mean(v_0..v_p) and lse = c + ln(p + 1), c = sm_scale * q . k."""
    g = torch.Generator().manual_seed(5)
    qo, kv, Hq, Hkv, D = [6, 1], [40, 23], 2, 1, 32
    ks, vs, qs = [], [], []
    for r in range(2):
        k1 = torch.randn(1, Hkv, D, generator=g).to(torch.bfloat16)
        ks.append(k1.expand(kv[r], Hkv, D).clone())
        vs.append(torch.randn(kv[r], Hkv, D, generator=g).to(torch.bfloat16))
        qs.append(torch.randn(qo[r], Hq, D, generator=g).to(torch.bfloat16))
    b = W.assemble_batch(qo, kv, qs, ks, vs, num_pages=16, batch_seed=4,
                         sm_scale=0.3)
    out, lse = _run(b)
    row = 0
    for r in range(2):
        for i in range(qo[r]):
            p = kv[r] - qo[r] + i
            for h in range(Hq):
                c = 0.3 * float(_f64(qs[r][i, h]) @ _f64(ks[r][0, 0]))
                _close(out[row, h], _f64(vs[r][: p + 1, 0]).mean(axis=0), TOL,
                       "identical keys: out = mean v")
                _close(lse[row, h], c + math.log(p + 1), TOL,
                       "identical keys: lse = c + ln(p+1)")
            row += 1


def load_three_token_golden():
    rows = []
    with open(os.path.join(HERE, "golden", "three_token_causal.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(x) for x in line.split()])
    return np.array(rows)


def three_token_batch(head_dim: int = 2) -> W.PagedBatch:
    """The hand example; ``head_dim > 2`` zero-pads q, k, v (which leaves the
    logits and the first two output dims unchanged)."""
    q = torch.zeros(3, 1, head_dim)
    q[:, 0, 0] = 1.0
    k = torch.zeros(3, 1, head_dim)
    k[:, 0, 0] = torch.tensor([0.0, 1.0, 2.0])
    v = torch.zeros(3, 1, head_dim)
    v[:, 0, :2] = torch.tensor([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    return W.assemble_batch([3], [3], [q], [k], [v], num_pages=4, batch_seed=9,
                            sm_scale=1.0)


def pin_hand_example():
    gold = load_three_token_golden()
    e = math.e
    closed = np.array([
        [0, 1.0, 0.0, 0.0],
        [1, 1 / (1 + e), e / (1 + e), math.log(1 + e)],
        [2, (1 + e * e) / (1 + e + e * e), (e + e * e) / (1 + e + e * e),
         math.log(1 + e + e * e)],
    ])
    _close(gold, closed, 1e-15, "golden file vs closed form")
    out, lse = _run(three_token_batch())
    _close(out[:, 0, :], gold[:, 1:3], TOL, "3-token example: out")
    _close(lse[:, 0], gold[:, 3], TOL, "3-token example: lse")


def dense_reference(b: W.PagedBatch):
    """Dense float64 attention from the contiguous copies (no page reads):
    ``scaled_dot_product_attention`` with an explicit bottom-right causal mask
    and ``enable_gqa`` (kv head h // group), lse from ``torch.logsumexp``."""
    outs, lses = [], []
    for r in range(b.batch):
        qo, kv = int(b.qo_lens()[r]), int(b.kv_lens()[r])
        if qo == 0:
            continue
        q = b.q[b.qo_indptr[r]: b.qo_indptr[r + 1]].double().transpose(0, 1)
        k = b.k_seq[r].double().transpose(0, 1)
        v = b.v_seq[r].double().transpose(0, 1)
        i = torch.arange(qo)[:, None]
        j = torch.arange(kv)[None, :]
        mask = j <= (kv - qo) + i
        o = torch.nn.functional.scaled_dot_product_attention(
            q, k, v, attn_mask=mask, scale=b.sm_scale, enable_gqa=True)
        group = b.num_qo_heads // b.num_kv_heads
        kr = k.repeat_interleave(group, dim=0)
        s = b.sm_scale * (q @ kr.transpose(1, 2))
        s = s.masked_fill(~mask, float("-inf"))
        outs.append(o.transpose(0, 1))
        lses.append(torch.logsumexp(s, dim=-1).transpose(0, 1))
    return torch.cat(outs).numpy(), torch.cat(lses).numpy()


def ragged_batch(page_size: int = 16) -> W.PagedBatch:
    """Ragged mix: decode-like, prefix + chunk, fresh prefill, empty query,
    lengths off the page size; 4 q heads over 2 kv heads."""
    reqs = [W.Request(1, 1, 21), W.Request(5, 37, 22), W.Request(16, 16, 23),
            W.Request(0, 20, 24), W.Request(17, 50, 25), W.Request(1, 33, 26)]
    return W.make_batch(reqs, num_qo_heads=4, num_kv_heads=2, head_dim=16,
                        num_pages=64, batch_seed=6, page_size=page_size,
                        keep_seq=True)


def pin_dense_library():
    for P in (16, 4):
        b = ragged_batch(P)
        out, lse = _run(b)
        ro, rl = dense_reference(b)
        _close(out, ro, 1e-12, f"dense library (P={P}): out")
        _close(lse, rl, 1e-12, f"dense library (P={P}): lse")


def pin_causal_library():
    """qo = kv (no prefix): the library's own causal mode, ``is_causal=True``."""
    b = W.make_batch([W.Request(40, 40, 31), W.Request(9, 9, 32)], num_qo_heads=2,
                     num_kv_heads=2, head_dim=8, num_pages=16, batch_seed=7,
                     keep_seq=True)
    out, _ = _run(b)
    for r in range(2):
        q = b.q[b.qo_indptr[r]: b.qo_indptr[r + 1]].double().transpose(0, 1)
        k = b.k_seq[r].double().transpose(0, 1)
        v = b.v_seq[r].double().transpose(0, 1)
        o = torch.nn.functional.scaled_dot_product_attention(
            q, k, v, is_causal=True, scale=b.sm_scale).transpose(0, 1)
        _close(out[b.qo_indptr[r]: b.qo_indptr[r + 1]], o.numpy(), 1e-12,
               "is_causal library")


def pin_merge():
    """Merging per-part states of a key partition equals attention over all
    keys (both from the library); empty parts change nothing; a row of only
    empty states gives (0, -inf)."""
    g = torch.Generator().manual_seed(8)
    H, D, n = 3, 16, 45
    q = torch.randn(H, 1, D, generator=g, dtype=torch.float64)
    k = torch.randn(H, n, D, generator=g, dtype=torch.float64)
    v = torch.randn(H, n, D, generator=g, dtype=torch.float64)
    scale = 0.4
    parts = [(0, 7), (7, 7), (7, 30), (30, 45)]
    vs, ss = [], []
    for lo, hi in parts:
        if hi == lo:
            vs.append(torch.zeros(H, D, dtype=torch.float64))
            ss.append(torch.full((H,), float("-inf"), dtype=torch.float64))
            continue
        o = torch.nn.functional.scaled_dot_product_attention(
            q, k[:, lo:hi], v[:, lo:hi], scale=scale)
        vs.append(o[:, 0])
        ss.append(torch.logsumexp(scale * (q @ k[:, lo:hi].transpose(1, 2)),
                                  dim=-1)[:, 0])
    full = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)
    full_lse = torch.logsumexp(scale * (q @ k.transpose(1, 2)), dim=-1)[:, 0]
    # row 0: all parts; row 1: one empty state only; row 2: one live state
    V = torch.stack(vs + [vs[1], vs[2]]).numpy()
    S = torch.stack(ss + [ss[1], ss[2]]).numpy()
    out, lse = A.merge_states(V, S, [0, 4, 5, 6])
    _close(out[0], full[:, 0].numpy(), 1e-12, "merge: out")
    _close(lse[0], full_lse.numpy(), 1e-12, "merge: lse")
    _close(out[1], np.zeros((H, D)), 0.0, "merge: all-empty out")
    assert np.all(lse[1] == -np.inf), "merge: all-empty lse"
    _close(out[2], vs[2].numpy(), 1e-15, "merge: single state out")
    _close(lse[2], ss[2].numpy(), 1e-15, "merge: single state lse")


def pin_chunk_and_decode_consistency():
    """A chunk over cached prefix pages gives the unchunked rows; a decode
    step gives the last prefill row."""
    seq = W.tiny_sequence()
    full_out, full_lse = _run(seq.batch)
    for lo, hi in ((128, 300), (100, 200), (299, 300), (0, 17)):
        o, l = _run(seq.chunk(lo, hi))
        _close(o, full_out[lo:hi], 1e-12, f"chunk [{lo},{hi}) out")
        _close(l, full_lse[lo:hi], 1e-12, f"chunk [{lo},{hi}) lse")
    d = seq.chunk(299, 300)
    o, l = A.decode_paged(d.q, d.k_pool, d.v_pool, d.kv_indptr, d.page_table,
                          d.num_kv_heads, d.sm_scale)
    _close(o[0], full_out[299], 1e-12, "decode = last prefill row")


def pin_page_relocation():
    """The same requests on other pages (data moved along) give the same
    result."""
    reqs = [W.Request(5, 37, 22), W.Request(17, 50, 25)]
    kw = dict(num_qo_heads=4, num_kv_heads=2, head_dim=16, num_pages=64)
    o1, l1 = _run(W.make_batch(reqs, batch_seed=1, **kw))
    o2, l2 = _run(W.make_batch(reqs, batch_seed=2, **kw))
    _close(o1, o2, 0.0, "relocated pages: out")
    _close(l1, l2, 0.0, "relocated pages: lse")


def pin_value_shift():
    """V + c gives out + c (softmax weights sum to one)."""
    b = ragged_batch()
    vp = b.v_pool.double().numpy()
    kp = b.k_pool.double().numpy()
    o1, _ = A.attention_paged(b.q, kp, vp, b.qo_indptr, b.kv_indptr, b.page_table,
                              b.num_kv_heads, b.sm_scale)
    o2, _ = A.attention_paged(b.q, kp, vp + 0.75, b.qo_indptr, b.kv_indptr,
                              b.page_table, b.num_kv_heads, b.sm_scale)
    live = ~np.isnan(o1)
    _close(o2[live], o1[live] + 0.75, 1e-12, "V + c")


def pin_gqa_is_repeated_mha():
    """GQA equals MHA whose kv heads are the GQA kv heads repeated per group
    (``repeat_interleave``: kv head h // group serves q head h)."""
    b = ragged_batch()
    group = b.num_qo_heads // b.num_kv_heads
    kp = b.k_pool.repeat_interleave(group, dim=2)
    vp = b.v_pool.repeat_interleave(group, dim=2)
    o1, l1 = _run(b)
    o2, l2 = A.attention_paged(b.q, kp, vp, b.qo_indptr, b.kv_indptr, b.page_table,
                               b.num_qo_heads, b.sm_scale)
    _close(o1, o2, 0.0, "GQA vs repeated MHA: out")
    _close(l1, l2, 0.0, "GQA vs repeated MHA: lse")


# ------------------------------------------------------------- latent (MLA) --

def _run_mla(b: W.PagedBatch, rows=None):
    return A.mla_attention_paged(b.q, b.k_pool, b.qo_indptr, b.kv_indptr, b.page_table,
                                 b.sm_scale, W.MLA_DV, rows=rows)


def pin_mla_one_key():
    """One visible key: out is the first 512 dims of that latent row, lse its
    scaled score over all 576 dims."""
    b = W.make_mla_batch([W.Request(1, 1, 41), W.Request(2, 2, 42)], num_qo_heads=4,
                         num_pages=8, batch_seed=9, keep_seq=True)
    out, lse = _run_mla(b)
    for r, row in ((0, 0), (1, 1)):    # request 1's first query sees its key 0 only
        kv0 = _f64(b.k_seq[r][0, 0])
        g = int(b.qo_indptr[r])
        _close(out[g, :, :], np.broadcast_to(kv0[:W.MLA_DV], (4, W.MLA_DV)), TOL,
               "MLA one key: out")
        q = _f64(b.q[g])
        _close(lse[g], b.sm_scale * (q @ kv0), TOL, "MLA one key: lse")


def pin_mla_identical_keys():
    """All latent rows equal: out is that row's first 512 dims and lse =
    s + ln(number of visible keys)."""
    kv_len, qo = 37, 5
    row = torch.randn(W.MLA_DK, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    kv = row.expand(kv_len, 1, W.MLA_DK).clone()
    q = torch.randn(qo, 2, W.MLA_DK, generator=torch.Generator().manual_seed(6))
    b = W.assemble_batch([qo], [kv_len], [q], [kv], [kv], num_pages=8, batch_seed=3,
                         sm_scale=1.0 / math.sqrt(192.0))
    b.v_pool = b.k_pool[..., :W.MLA_DV]
    out, lse = _run_mla(b)
    r64 = _f64(row)
    qd = _f64(b.q)
    for i in range(qo):
        n_vis = kv_len - qo + i + 1
        _close(out[i], np.broadcast_to(r64[:W.MLA_DV], (2, W.MLA_DV)), TOL,
               "MLA identical keys: out")
        _close(lse[i], b.sm_scale * (qd[i] @ r64) + math.log(n_vis), TOL,
               "MLA identical keys: lse")


def pin_mla_dense():
    """Dense float64 library attention over the contiguous latent rows (no page
    reads): every q head against the one shared row, values its first 512
    dims, explicit bottom-right causal mask."""
    reqs = [W.Request(1, 40, 51), W.Request(6, 23, 52), W.Request(17, 17, 53),
            W.Request(0, 9, 54)]
    b = W.make_mla_batch(reqs, num_qo_heads=8, num_pages=32, batch_seed=11, keep_seq=True)
    out, lse = _run_mla(b)
    for r in range(b.batch):
        qo, kv = int(b.qo_lens()[r]), int(b.kv_lens()[r])
        if qo == 0:
            continue
        q = b.q[b.qo_indptr[r]: b.qo_indptr[r + 1]].double().transpose(0, 1)  # [H, qo, Dk]
        k = b.k_seq[r][:, 0].double()                                            # [kv, Dk]
        i = torch.arange(qo)[:, None]
        j = torch.arange(kv)[None, :]
        mask = j <= (kv - qo) + i
        o = torch.nn.functional.scaled_dot_product_attention(
            q, k.expand(8, kv, W.MLA_DK), k[:, :W.MLA_DV].expand(8, kv, W.MLA_DV),
            attn_mask=mask, scale=b.sm_scale)
        s = (b.sm_scale * (q @ k.T)).masked_fill(~mask, float("-inf"))
        g0 = int(b.qo_indptr[r])
        _close(out[g0: g0 + qo], o.transpose(0, 1).numpy(), 1e-12, "MLA dense: out")
        _close(lse[g0: g0 + qo], torch.logsumexp(s, dim=-1).T.numpy(), 1e-12, "MLA dense: lse")


ALL_PINS = [pin_one_key, pin_identical_keys, pin_hand_example, pin_dense_library,
            pin_causal_library, pin_merge, pin_chunk_and_decode_consistency,
            pin_page_relocation, pin_value_shift, pin_gqa_is_repeated_mha,
            pin_mla_one_key, pin_mla_identical_keys, pin_mla_dense]


def failing_pins():
    """Names of the pins that fail (for the planted-mistake test)."""
    failed = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    return failed
