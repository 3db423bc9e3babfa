"""CPU oracle of the block token-eviction hot path — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct float64 implementations (numpy) of the six
operations of the path, written from the pages' definitions:

* ``focus_importance_delta`` — FOCUS importance I_j and delta Delta-I
  (FOCUS paper, arXiv 2601.23278: Section 3.1 Eq. 2, Section 3.2 Eq. 3,
  Section 4.2; App. E.2.1; FOCUS notes page, key design 1).
* ``esdllm_score`` — ES-dLLM importance score (ES-dLLM notes page, key
  design 1); ``esdllm_skip_layer`` — one skip layer of its early skipping
  (score, partial hidden-cache update, top-(1-r)|S|, survivor compaction;
  key designs 1 and 2), ``esdllm_skip_layer_ragged`` the same on survivor
  sets of per-sequence size; ``esdllm_schedule`` — the per-sequence iteration
  bookkeeping (initial full pass, periodic refresh without skipping, survivor
  reset; key design 2); ``esdllm_iteration`` — both composed.
* ``topk_select`` — per-sequence top-K of masked tokens (FOCUS paper
  Section 4.2; ES-dLLM notes page, key design 1 "top-(1-r_l)|S|").
* ``gather_rows`` — Gather of the kept block hidden rows into H_reduced
  (FOCUS paper Section 4.2; App. E.2.3 prefix-sum compaction).
* ``kv_scatter`` — in-place scatter of the kept rows' new K/V into the
  exact KV cache (ES-dLLM notes page, key design 2; FOCUS paper App. E.2.4).
* ``reduced_attention`` — attention of the kept queries over prefix plus
  block KV (FOCUS paper Section 2, Section 4.2; App. E.2.4).
* ``focus_budget``, ``history_update`` — FOCUS dynamic budget K and its
  per-sequence history (FOCUS notes page, key design 2; FOCUS paper
  Section 4.1, App. E.3.1).
* ``focus_select`` — top-K plus FOCUS's structural constraints (AR-context,
  placeholder integrity, |S| >= 1; FOCUS paper Section 4.2, App. E.2.2).
* ``kv_scatter_paged``, ``reduced_attention_paged`` — the same scatter and
  attention on a paged KV pool through a page table (FOCUS paper App. E.2.4).
* ``commit_mask`` — the neighbour-aware delayed commit of block KV states
  (FOCUS paper Section 4.3, App. E.3.1, App. E.3.3).
* ``gather_rows_multi`` — several row tensors compacted with one index set
  (FOCUS paper App. E.2.3); ``gather_rows_ragged`` — a gather from sources
  compacted by sequence.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path
(``block_token_eviction_amd``) never imports, links or calls it, and this
package shares no code with the HIP kernels.

Every function is pinned by tests in ``tests/test_oracle_*.py`` against
closed forms, hand-worked examples, library routines and invariants.
"""
from .focus import (block_scores, maxpool_keys, softmax_keys, importance,
                    focus_importance_delta)
from .esdllm import (esdllm_score, esdllm_skip_layer, esdllm_schedule, esdllm_skip_layer_ragged,
                     esdllm_iteration)
from .selection import topk_select, focus_select
from .budget import focus_budget, history_update
from .rows import gather_rows, gather_rows_multi, gather_rows_ragged, kv_scatter
from .cache_state import commit_mask
from .attention import reduced_attention
from .paged import kv_scatter_paged, reduced_attention_paged, physical_row

__all__ = ["block_scores", "maxpool_keys", "softmax_keys", "importance",
           "focus_importance_delta", "esdllm_score", "topk_select", "gather_rows",
           "kv_scatter", "reduced_attention", "focus_budget",
           "history_update", "focus_select", "kv_scatter_paged", "reduced_attention_paged",
           "physical_row", "commit_mask", "gather_rows_multi", "esdllm_skip_layer",
           "esdllm_schedule", "esdllm_skip_layer_ragged", "esdllm_iteration", "gather_rows_ragged"]
