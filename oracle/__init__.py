"""CPU float64 oracle for deterministic paged attention — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product library never calls it and
shares no code with it.

What it computes is the plain definition of causal softmax attention over a
paged KV cache, the result that split-KV prefill and decode with a fixed-order
merge of partial (o, lse) states reach in exact arithmetic (sglang PR #10417
"[POC] Support deterministic inference", Modifications: paged prefill wrapper
for every extend, fixed split-KV of 2048 for decode and 4096 for prefill;
sglang PR #43612, Summary: a chunked prefill over the cached prefix must equal
the unchunked call).

Every function here is pinned by ``tests/test_oracle_pins.py`` against closed
forms, a hand example, a dense library computation and exact invariances, and
``tests/test_oracle_mutations.py`` shows that planted mistakes fail those pins.
"""
from .attention import (attend, attention_paged, decode_paged, gather_request_kv,
                        kv_head_of, latent_values, merge_states, mla_attention_paged,
                        page_offsets, query_position)

__all__ = ["attend", "attention_paged", "decode_paged", "gather_request_kv",
           "kv_head_of", "latent_values", "merge_states", "mla_attention_paged",
           "page_offsets", "query_position"]
