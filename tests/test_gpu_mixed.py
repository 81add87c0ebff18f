"""The mixed long-context workload: one 65536-token request prefilled in four
16384-token chunks (on the 128-token grid, over its cached prefix pages) must
reproduce the unchunked 65536-token call bit for bit (sglang PR #43612,
Summary), and every chunk meets oracle parity on a fixed row sample."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import assert_parity, bits_equal, run_prefill, sample_rows, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_65536_in_four_chunks_equals_unchunked():
    seq = W.make_sequence(65536, seed=5, num_pages=8192, device=DEV)
    say("mixed: unchunked 65536-token prefill (split 4096)")
    full, full_lse = run_prefill(seq.batch)
    assert torch.isfinite(full.float()).all() and torch.isfinite(full_lse).all()
    for lo, hi in W.chunk_bounds(65536, 16384):
        say(f"mixed: chunk [{lo}, {hi})")
        ch = seq.chunk(lo, hi)
        out, lse = run_prefill(ch)
        assert bits_equal(out, full[lo:hi]), f"chunk [{lo}, {hi}) out differs from unchunked"
        assert bits_equal(lse, full_lse[lo:hi]), f"chunk [{lo}, {hi}) lse differs"
        rows = {0: sample_rows(hi - lo, edge=32, every=1021)}
        assert_parity(out, lse, ch, [0], rows, what=f"mixed chunk [{lo}, {hi}) (sampled)")
