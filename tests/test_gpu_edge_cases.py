"""Edge cases of the online softmax on the GPU, against the float64 oracle
and closed forms.

* A key whose logit leaps about 155 base-2 units above every earlier key of
  the row: exp2 of the score against the stale running max overflows to
  inf, which must make the row take the tile max and recompute (prefill), or
  raise its max (decode), and give a finite result equal to the oracle's.
* Identical keys: every row's output is the mean of the values it sees and
  its lse is the common logit plus ln(number of keys) (a closed form of the
  definition, independent of the oracle)."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import (LSE_TOL, OUT_TOL, assert_parity, run_decode, run_prefill, say)

pytestmark = pytest.mark.gpu
DEV = "cuda"

HEADS = [W.QWEN3_8B, dict(num_qo_heads=4, num_kv_heads=1, head_dim=64)]
IDS = ["hq32_hkv8_d128", "hq4_hkv1_d64"]


@pytest.mark.parametrize("heads", HEADS, ids=IDS)
@pytest.mark.parametrize("split", [256, 4096])
def test_logit_jump_prefill(heads, split):
    # jumps mid-tile, at a tile's first key, in a later partition, and in a
    # chunk whose prefix holds the jump
    qo = [1500, 700, 900, 300]
    kv = [1500, 700, 3000, 1200]
    jump = [1000, 320, 2600, 100]
    say(f"logit jump prefill {heads} split {split}")
    b = W.jump_batch(qo, kv, jump, seed=71, num_pages=1024, device=DEV, **heads)
    out, lse = run_prefill(b, split=split)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    # rows at or past the jump see a logit far above the rest
    assert float(lse.max()) > 60.0
    assert_parity(out, lse, b, what=f"logit jump prefill split {split}")


@pytest.mark.parametrize("heads", HEADS, ids=IDS)
def test_logit_jump_decode(heads):
    ctx = [1, 300, 2049, 5000, 9000]
    jump = [0, 299, 1, 4100, 64]
    say(f"logit jump decode {heads}")
    b = W.jump_batch([1] * len(ctx), ctx, jump, seed=72, num_pages=2048, device=DEV, **heads)
    out, lse = run_decode(b)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    assert_parity(out, lse, b, what="logit jump decode")


def _closed_form(b, r, mode):
    """Mean of the visible values and c + ln(p + 1), float64, for request r."""
    g = b.num_qo_heads // b.num_kv_heads
    qo, kv = int(b.qo_lens()[r]), int(b.kv_lens()[r])
    q = b.q[int(b.qo_indptr[r]): int(b.qo_indptr[r + 1])].double().cpu().numpy()
    w = b.k_seq[r][0].double().numpy()            # [Hkv, D], every key equals it
    v = b.v_seq[r].double().numpy()               # [kv, Hkv, D]
    csum = np.cumsum(v, axis=0)
    out = np.zeros((qo, b.num_qo_heads, b.head_dim))
    lse = np.zeros((qo, b.num_qo_heads))
    for i in range(qo):
        p = kv - qo + i
        for h in range(b.num_qo_heads):
            hk = h // g
            out[i, h] = csum[p, hk] / (p + 1)
            lse[i, h] = b.sm_scale * float(q[i, h] @ w[hk]) + math.log(p + 1)
    return out, lse


@pytest.mark.parametrize("heads", HEADS, ids=IDS)
@pytest.mark.parametrize("mode", ["prefill", "decode"])
def test_identical_keys_closed_form(heads, mode):
    if mode == "prefill":
        qo, kv = [1, 200, 500, 129], [1, 200, 2100, 4200]
    else:
        qo, kv = [1, 1, 1, 1], [1, 77, 2048, 6000]
    say(f"identical keys {mode} {heads}")
    b = W.identical_keys_batch(qo, kv, seed=73, num_pages=1024, device=DEV, **heads)
    out, lse = run_prefill(b, split=1024) if mode == "prefill" else run_decode(b)
    for r in range(b.batch):
        o_ref, l_ref = _closed_form(b, r, mode)
        rows = slice(int(b.qo_indptr[r]), int(b.qo_indptr[r + 1]))
        e_out = float(np.max(np.abs(out[rows].double().cpu().numpy() - o_ref)))
        e_lse = float(np.max(np.abs(lse[rows].double().cpu().numpy() - l_ref)))
        say(f"  request {r}: max|out - mean(v)| {e_out:.3e}  max|lse - (c + ln n)| {e_lse:.3e}")
        assert e_out <= OUT_TOL and e_lse <= LSE_TOL
    assert_parity(out, lse, b, what=f"identical keys {mode}")
