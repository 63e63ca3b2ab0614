"""Oracle attention and LSE merge in float64 (test infrastructure only).

Layout convention (the pages are silent on it): Q, K, V and the output are
``[B, S, H, D]`` arrays (batch, sequence, heads, head_dim); the LSE is
``[B, H, Sq]``.  The LSE is the natural logarithm of the softmax denominator,
with the scale inside: ``lse_i = ln sum_j exp(scale * q_i . k_j)``.

Attention is non-causal with no mask, no dropout and no bias: the Ring
Anything variant is inference-only and requires ``attn_mask`` to be ``None``
(context-parallelism guide, "Paralelisme konteks", diffusers v0.43.0, section
"Ring Anything Attention"), and the ring shard of a diffusion transformer
attends bidirectionally.
"""

from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np


def _as_f64(x) -> np.ndarray:
    a = np.asarray(x, dtype=np.float64)
    if a.ndim != 4:
        raise ValueError(f"expected a [B, S, H, D] array, got shape {a.shape}")
    return a


def attention_fp64(q, k, v, scale: float, row_block: int = 1024) -> Tuple[np.ndarray, np.ndarray]:
    """One-shot softmax attention of every query row over every key.

    For each batch b, head h and query row i::

        s_j   = scale * sum_d q[b,i,h,d] * k[b,j,h,d]      (all keys j, in order)
        m     = max_j s_j
        lse   = m + ln sum_j exp(s_j - m)
        out_d = sum_j exp(s_j - lse) * v[b,j,h,d]

    This is the result every rank of the ring reaches once it has seen the K/V
    of every token (guide, section "Ring Attention").  Query rows are
    independent, so they are processed in blocks of ``row_block`` rows only to
    bound memory.  With zero keys the result is the merge identity:
    ``out = 0`` and ``lse = -inf``.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, Sq, H, D = q.shape
    if k.shape[0] != B or k.shape[2] != H or k.shape[3] != D or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    Skv = k.shape[1]
    scale = float(scale)
    out = np.zeros((B, Sq, H, D), dtype=np.float64)
    lse = np.full((B, H, Sq), -np.inf, dtype=np.float64)
    if Skv == 0:
        return out, lse
    for b in range(B):
        for h in range(H):
            kh = k[b, :, h, :]          # [Skv, D]
            vh = v[b, :, h, :]          # [Skv, D]
            for r0 in range(0, Sq, row_block):
                r1 = min(Sq, r0 + row_block)
                qh = q[b, r0:r1, h, :]  # [rows, D]
                s = scale * (qh @ kh.T)  # [rows, Skv]
                m = s.max(axis=1)
                row_lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
                weights = np.exp(s - row_lse[:, None])
                out[b, r0:r1, h, :] = weights @ vh
                lse[b, h, r0:r1] = row_lse
    return out, lse


def attention_rows_fp64(q, k, v, scale: float, rows: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """``attention_fp64`` restricted to the query rows ``rows`` (all heads).

    Returns ``out[B, len(rows), H, D]`` and ``lse[B, H, len(rows)]``; used to
    check full-size GPU results on a sample of rows.
    """
    q = _as_f64(q)
    idx = np.asarray(list(rows), dtype=np.int64)
    return attention_fp64(q[:, idx], k, v, scale)


def chunk_partial_fp64(q, k_chunk, v_chunk, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """The partial result of attending to one K/V chunk: that chunk's own
    normalised output and LSE.  An empty chunk gives the merge identity
    (``out = 0``, ``lse = -inf``)."""
    return attention_fp64(q, k_chunk, v_chunk, scale)


def lse_merge_fp64(out_a, lse_a, out_b, lse_b) -> Tuple[np.ndarray, np.ndarray]:
    """Merge two partial attention results by their log-sum-exp weights.

    The pages state that ring attention keeps the output and LSE in float32
    for numerical stability (Parallelism API page,
    ``ContextParallelConfig.convert_to_fp32``) but do not print the merge.
    The reading taken is the exact combination of two softmax partials over
    disjoint key sets, written in max-shifted form::

        lse = max(a, b) + ln(1 + exp(-|a - b|))
        out = exp(a - lse) * out_a + exp(b - lse) * out_b

    A partial with ``lse = -inf`` (an empty key set) contributes nothing and is
    never multiplied, so garbage in its output cannot leak; if both are empty
    the result is the identity ``(0, -inf)``.

    ``out_*`` are ``[B, Sq, H, D]``; ``lse_*`` are ``[B, H, Sq]``.
    """
    out_a = np.asarray(out_a, dtype=np.float64)
    out_b = np.asarray(out_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    B, H, Sq = lse_a.shape
    out = np.zeros_like(out_a)
    lse = np.full_like(lse_a, -np.inf)
    for b in range(B):
        for h in range(H):
            for i in range(Sq):
                a = lse_a[b, h, i]
                c = lse_b[b, h, i]
                if a == -np.inf and c == -np.inf:
                    continue
                if a == -np.inf:
                    out[b, i, h, :] = out_b[b, i, h, :]
                    lse[b, h, i] = c
                    continue
                if c == -np.inf:
                    out[b, i, h, :] = out_a[b, i, h, :]
                    lse[b, h, i] = a
                    continue
                new = max(a, c) + math.log1p(math.exp(-abs(a - c)))
                out[b, i, h, :] = math.exp(a - new) * out_a[b, i, h, :] + math.exp(c - new) * out_b[b, i, h, :]
                lse[b, h, i] = new
    return out, lse


def ring_shard_fp64(q, k, v, offsets: Sequence[int], scale: float,
                    order: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """One rank's ring attention computed the ring's way: attend the local Q to
    each K/V chunk ``[offsets[c], offsets[c+1])`` in turn (``order``, default
    0..N-1, the all-gather order of the API page's ``rotate_method``) and fold
    each chunk partial into the running result with ``lse_merge_fp64``
    (guide, section "Ring Attention"; API page, ``ring_degree`` and
    ``convert_to_fp32``).  Used only to pin the merge against the one-shot
    definition."""
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    n = len(offsets) - 1
    if order is None:
        order = range(n)
    B, Sq, H, D = q.shape
    out = np.zeros((B, Sq, H, D))
    lse = np.full((B, H, Sq), -np.inf)
    for c in order:
        lo, hi = offsets[c], offsets[c + 1]
        part_out, part_lse = chunk_partial_fp64(q, k[:, lo:hi], v[:, lo:hi], scale)
        out, lse = lse_merge_fp64(out, lse, part_out, part_lse)
    return out, lse


def ulysses_head_range(n_heads: int, ulysses_degree: int, rank: int) -> Tuple[int, int]:
    """Heads ``[lo, hi)`` that rank ``rank`` holds after the Ulysses all-to-all:
    every token for an even share of the heads.  The head count must divide by
    the degree (guide, variant table and section "Perhatian Ulysses")."""
    if ulysses_degree < 1 or not 0 <= rank < ulysses_degree:
        raise ValueError("bad ulysses degree / rank")
    if n_heads % ulysses_degree != 0:
        raise ValueError(f"{n_heads} heads do not divide by ulysses_degree {ulysses_degree}")
    per = n_heads // ulysses_degree
    return rank * per, (rank + 1) * per


def _round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even) and return
    them as float64; -inf stays -inf."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to(torch.bfloat16).to(torch.float64).numpy()


def ring_shard_bf16_state_fp64(q, k, v, offsets: Sequence[int], scale: float,
                               order: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """The ring's way with the merge state kept in bf16 -- the mode that
    ContextParallelConfig.convert_to_fp32 = False selects (Parallelism API
    page: without it the output and LSE are not converted to float32 for the
    merge).  Each chunk partial (output, LSE) is rounded to bf16, merged with
    the stored state by the LSE formula in float64, and the merged state is
    rounded to bf16 again.  Only used to measure the error that the float32
    merge avoids."""
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    n = len(offsets) - 1
    if order is None:
        order = range(n)
    B, Sq, H, D = q.shape
    out = np.zeros((B, Sq, H, D))
    lse = np.full((B, H, Sq), -np.inf)
    for c in order:
        lo, hi = offsets[c], offsets[c + 1]
        part_out, part_lse = chunk_partial_fp64(q, k[:, lo:hi], v[:, lo:hi], scale)
        part_out, part_lse = _round_bf16(part_out), _round_bf16(part_lse)
        out, lse = lse_merge_fp64(out, lse, part_out, part_lse)
        out, lse = _round_bf16(out), _round_bf16(lse)
    return out, lse
