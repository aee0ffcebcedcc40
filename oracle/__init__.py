"""Plain fp64 CPU oracle for zigzag ring context-parallel attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` use it.  It shares no code with the HIP library (no kernels,
headers, helpers or constant tables); both sides receive the same seeded
inputs from ``ring_context_parallelism_amd.inputs``, which holds no part of the
method's arithmetic.

Sources (pages, cited by title and section):

* "Sequence Parallelism IV: Megatron Context Parallel and Load-Balanced
  Rings" (duoan.github.io) -- the method: Q stays local while K/V chunks
  circulate (section 4 "What Actually Moves"), exact online-softmax merging of
  partial results (section 4), zigzag ``2*cp`` chunk placement pairing early and
  late chunks (section 3 "Naive Ring Attention Is Imbalanced Under Causal
  Masks"), per-iteration work balance (section 3).
* "Context Parallelism in MegaDLMs: How It Handles Long Sequences"
  (instagit.com) -- per-GPU length ``seq_length // context_parallel_size``
  (section "Sequence Partitioning Across GPUs").
* "Context Parallelism for Long-Context Training" (jpcasabianca.com) --
  equivalence against the unsharded reference for outputs and gradients
  (section "Prove attention equivalence"; the gradients in ``backward``), shard coverage and padding of awkward lengths (section "Test
  sequence divisibility and padding": pad ownership, masked pad keys and
  queries, real outputs unchanged by the padding).

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, invariants, brute force or an independent library
routine; none is "parity unpinned".
"""

from .attention import attention, attention_probabilities, document_of, valid_mask
from .backward import attention_backward, query_gradients, rank_backward, full_backward
from .cp_reference import (
    chunk_size,
    padded_length,
    rank_chunks,
    rank_positions,
    ring_source,
    merge_partial,
    rank_forward,
    full_forward,
    sequence_shards,
    head_shards,
    ulysses_forward,
    step_valid_pairs,
    step_valid_tiles,
    imbalance,
    valid_flops,
)

__all__ = [
    "attention",
    "attention_probabilities",
    "valid_mask",
    "document_of",
    "attention_backward",
    "query_gradients",
    "rank_backward",
    "full_backward",
    "chunk_size",
    "padded_length",
    "rank_chunks",
    "rank_positions",
    "ring_source",
    "merge_partial",
    "rank_forward",
    "full_forward",
    "sequence_shards",
    "head_shards",
    "ulysses_forward",
    "step_valid_pairs",
    "step_valid_tiles",
    "imbalance",
    "valid_flops",
]
