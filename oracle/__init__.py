"""Plain float64 CPU oracle for head-wise sparse decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (``head_wise_sparse_02_amd``) and imports nothing from it.

Sources cited in this package (gist.science summary pages; titles as shown
on each page, the first one translated from Arabic):

* [RTPurbo] "Full attention returns in force: converting full attention to
  sparse attention within hundreds of training steps" (arXiv 2605.16928).
* [ICS] "Inference-time context sparsity: illusion or opportunity?"
  (arXiv 2605.24168).
* [NHA] "Native Hybrid Attention for Efficient Sequence Modeling"
  (arXiv 2510.07019).
* [AoH] "Autonomy-of-Heads: Data-Free Sparse Attention from Frozen Query-Key
  Geometry" (arXiv 2608.06849).

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, brute force, invariants or an independent library
routine.  The pages print no worked numeric example, so no stored value
comes from them.
"""

from .hws_oracle import (  # noqa: F401
    E4M3_MAX,
    bf16_round,
    decode_head_ref,
    decode_sequence_ref,
    e4m3_decode,
    effective_rank,
    e4m3_encode,
    e4m3_table,
    fp8_store_rows,
    full_logits,
    group_aggregate,
    head_probs,
    index_keys,
    index_logits,
    local_token_set,
    prefill_mask,
    prefill_sequence_ref,
    rope,
    select_top_k,
    select_top_p,
    sparse_attend,
    stored_rows,
)
