"""Plain, slow, fp64 CPU oracle for batched attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY. Nothing in the product package may import, call or
execute anything here. The only permitted users are ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``.

The oracle shares no code with the HIP path: it has its own dtype decoding,
its own page-table walk, its own attention-state arithmetic and its own copy of
the work-chunk rule. Its inputs are NumPy arrays (fp16 / bf16 values arrive as
raw uint16 bit patterns and are decoded here, exactly, to float64).

Sources (the FlashInfer pages: the aiwiki.ai article "FlashInfer" and the
docs.flashinfer.ai index "Welcome to FlashInfer's documentation!"):

* attention as exact softmax(q k^T * scale) v with a running maximum, the
  attention state (output, log-sum-exp) and its merge:
  article "FlashInfer", sections "Attention states" and
  "Extreme-negative-logit correction";
* the paged (block-sparse) cache with a page table:
  article "FlashInfer", section "Block-sparse cache representation";
* the host-side plan that splits the KV into work chunks:
  article "FlashInfer", section "Plan and run".
* appending new K/V rows into the paged cache: docs index "flashinfer.page" >
  "Append new K/V tensors to Paged KV-Cache", with the page walk above.
* block-sparse attention: docs index "flashinfer.sparse" >
  "BlockSparseAttentionWrapper", with exact attention over a block mask.
* attention variants (sliding window, logit soft cap, attention sinks), named
  in the article "FlashInfer", section "Custom attention templates"; their
  formulas are this oracle's readings, stated in ``variants.py``.

Every function is pinned by tests under ``tests/`` (brute force on tiny inputs,
closed forms, invariants, hand-worked golden fixtures). No function here is
"parity unpinned".
"""

from .attention import (  # noqa: F401
    NEG_INF,
    decode_bits,
    request_kv_len,
    request_token_pages,
    gather_request_kv,
    attention_state,
    single_decode,
    batch_decode,
    batch_prefill,
    merge_state,
    merge_states,
    cascade_decode,
)
from .plan import plan_spec, PlanSpec  # noqa: F401
from .append import append_positions, append_paged_kv  # noqa: F401
from .block_sparse import block_mask, block_sparse_attention  # noqa: F401
from .variants import (  # noqa: F401
    capped_logits,
    window_visible,
    variant_state,
    batch_decode_variant,
    batch_prefill_variant,
)
