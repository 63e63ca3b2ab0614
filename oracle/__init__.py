"""Plain CPU fp64 oracle for one GPU's share of ring attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package; only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code,
headers, tables or helpers with the HIP library and imports nothing from it.

What it computes, and where that is defined:

* ``chunk_offsets`` -- how a sequence of S tokens is split into N ring chunks,
  evenly for plain ring attention and unevenly for Ring Anything.
  Context-parallelism guide ("Paralelisme konteks", diffusers v0.43.0):
  the variant table at the top of the page and the section "Ring Anything
  Attention"; Parallelism API page, ``ContextParallelConfig.ring_anything``.
* ``attention_fp64`` -- one-shot non-causal softmax attention of a local Q shard
  over every key, returning the fp64 output and natural-log LSE.  After one
  full turn of the ring every GPU has attended to the K/V of every token
  (guide, section "Ring Attention"), so the ring shard's exact result is this
  plain definition.
* ``chunk_partial_fp64`` / ``lse_merge_fp64`` / ``ring_shard_fp64`` -- the
  per-chunk partial (output, LSE) and the log-sum-exp merge that
  ``ContextParallelConfig.convert_to_fp32`` keeps in float32 on the GPU.  The
  pages give the purpose of the merge but do not print its formula; the
  oracle uses the exact LSE-weighted combination (see ``lse_merge_fp64``).
* ``ring_shard_bf16_state_fp64`` -- the ring with its merge state kept in
  bf16 (``convert_to_fp32 = False``), to measure the error the float32
  merge avoids.
* ``brute_force_attention`` -- the same definition in pure-Python loops with
  ``math.fsum`` for tiny shapes.
* ``ulysses_head_range`` -- the head subset one GPU holds after the Ulysses
  all-to-all (guide, section "Perhatian Ulysses").
* ``cp_share`` / ``cp_mesh`` -- one rank's layout in the ring x Ulysses grid
  (Unified attention, Ulysses Anything, Ring Anything): its tokens before the
  all-to-all and the query rows and heads of its attention share (guide,
  sections "Perhatian Terpadu", "Ulysses Anything Attention"; API page,
  ``ContextParallelConfig``).

Every function here is pinned by a test in ``tests/test_oracle.py`` to
something other than itself (closed forms, a library routine, brute force,
invariants).  No function is parity unpinned.
"""

from .offsets import chunk_offsets, chunk_lengths, padded_chunk_length, pad_gather_slice
from .partition import cp_mesh, cp_share
from .attention import (
    attention_fp64,
    attention_rows_fp64,
    chunk_partial_fp64,
    lse_merge_fp64,
    ring_shard_fp64,
    ring_shard_bf16_state_fp64,
    ulysses_head_range,
)
from .brute import brute_force_attention

__all__ = [
    "chunk_offsets",
    "chunk_lengths",
    "padded_chunk_length",
    "pad_gather_slice",
    "attention_fp64",
    "attention_rows_fp64",
    "chunk_partial_fp64",
    "lse_merge_fp64",
    "ring_shard_fp64",
    "ring_shard_bf16_state_fp64",
    "ulysses_head_range",
    "brute_force_attention",
    "cp_mesh",
    "cp_share",
]
