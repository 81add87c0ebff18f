"""Planted mistakes in the CPU oracle must fail at least one pin.

Each case swaps one function of ``oracle.attention`` (on the CPU, for this
test only) for a copy with a plausible bug: a wrong index, a dropped term, a
wrong sign, a transposed operand. If no pin failed, the pins would not be
pinning that part of the oracle.
"""
import math

import numpy as np
import pytest

import oracle.attention as A
import oracle_pins


def _attend_variant(scale_on=True, log_base=math.e, normalise=True, swap_kv=False,
                    strict=False, drop_max=False):
    def attend(q_rows, K, V, positions, sm_scale):
        if swap_kv:
            K, V = V, K
        S = (sm_scale if scale_on else 1.0) * (q_rows @ K.T)
        j = np.arange(K.shape[0])[None, :]
        vis = (j < positions[:, None]) if strict else (j <= positions[:, None])
        S = np.where(vis, S, -np.inf)
        m = S.max(axis=1)
        l = np.exp(S - m[:, None]).sum(axis=1)
        lse = (0.0 if drop_max else m) + np.log(l) / math.log(log_base)
        if normalise:
            out = np.exp(S - (m + np.log(l))[:, None]) @ V
        else:
            out = np.exp(S - m[:, None]) @ V
        return out, lse
    return attend


def _gather_swapped(pool, page_table, page_off, kv_len, h_kv):
    P = pool.shape[1]
    rows = []
    for j in range(kv_len):
        page = int(page_table[page_off + j % P]) if page_off + j % P < len(page_table) \
            else int(page_table[-1])
        rows.append(A._page_rows(pool, page, h_kv)[(j // P) % P])
    return np.array(rows).reshape(kv_len, pool.shape[3])


def _page_offsets_floor(kv_lens, page_size):
    off = np.zeros(len(kv_lens), dtype=np.int64)
    total = 0
    for r, n in enumerate(kv_lens):
        off[r] = total
        total += int(n) // page_size
    return off


def _merge_variant(sign=1.0, divide=True, add_max=True):
    def merge_states(v, s, state_indptr):
        v = np.asarray(v, dtype=np.float64)
        s = np.asarray(s, dtype=np.float64)
        n_rows = len(state_indptr) - 1
        H, D = v.shape[1], v.shape[2]
        out = np.zeros((n_rows, H, D))
        lse = np.full((n_rows, H), -np.inf)
        for i in range(n_rows):
            lo, hi = state_indptr[i], state_indptr[i + 1]
            for h in range(H):
                si = s[lo:hi, h]
                live = si != -np.inf
                if not live.any():
                    continue
                M = si[live].max()
                w = np.exp(sign * (si[live] - M))
                acc = (w[:, None] * v[lo:hi, h][live]).sum(axis=0)
                out[i, h] = acc / w.sum() if divide else acc
                lse[i, h] = (M if add_max else 0.0) + math.log(w.sum())
        return out, lse
    return merge_states


MUTATIONS = {
    "gqa_head_modulo": ("kv_head_of", lambda h, group: h % group),
    "causal_top_left": ("query_position", lambda i, qo, kv: i),
    "causal_drops_diagonal": ("query_position", lambda i, qo, kv: kv - qo + i - 1),
    "causal_one_extra_key": ("query_position", lambda i, qo, kv: kv - qo + i + 1),
    "page_offsets_floor": ("page_offsets", _page_offsets_floor),
    "gather_page_slot_swapped": ("gather_request_kv", _gather_swapped),
    "no_softmax_scale": ("attend", _attend_variant(scale_on=False)),
    "lse_base2": ("attend", _attend_variant(log_base=2.0)),
    "out_not_normalised": ("attend", _attend_variant(normalise=False)),
    "k_and_v_swapped": ("attend", _attend_variant(swap_kv=True)),
    "mask_strict": ("attend", _attend_variant(strict=True)),
    "lse_drops_max": ("attend", _attend_variant(drop_max=True)),
    "merge_weight_sign": ("merge_states", _merge_variant(sign=-1.0)),
    "merge_no_division": ("merge_states", _merge_variant(divide=False)),
    "merge_lse_drops_max": ("merge_states", _merge_variant(add_max=False)),
    "mla_values_from_rope_end": ("latent_values", lambda kv, v_dim: kv[..., -v_dim:]),
    "mla_values_skip_first_dim": ("latent_values", lambda kv, v_dim: kv[..., 1:v_dim + 1]),
}


def test_unmutated_oracle_passes_every_pin():
    assert oracle_pins.failing_pins() == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_fails_a_pin(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(A, attr, bad)
    failed = oracle_pins.failing_pins()
    assert failed, f"no pin caught the planted mistake {name!r}"
