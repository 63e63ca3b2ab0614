"""Oracle side of the context-parallel layout of one rank (test
infrastructure only): which tokens a rank holds, and the query rows and heads
of its attention share, for ring, Ring Anything, Ulysses, Ulysses Anything
and Unified (ring x Ulysses) attention.

Sources (context parallelism guide "Paralelisme konteks", diffusers v0.43.0;
Parallelism API page, ContextParallelConfig):

* Unified attention ("Perhatian Terpadu"): the GPUs form a 2D grid of
  ulysses_degree x ring_degree; every GPU is in one Ulysses group and one ring
  group.  An all-to-all inside the Ulysses group regroups tokens and heads,
  ring attention runs over the ring group, and the inverse all-to-all
  restores the layout.
* Ulysses ("Perhatian Ulysses"): after the all-to-all a GPU holds every token
  of its group for a subset of the heads.
* Ulysses Anything: lifts the rule that the sequence length and the head
  count divide by ulysses_degree; needs ring_degree 1.  Ring Anything: any
  sequence length; needs ulysses_degree 1 (API page).
* ContextParallelConfig.mesh: a mesh with dims "ring" and "ulysses".

Readings where the pages are silent: the mesh is row-major over
("ring", "ulysses"), so rank = r * U + u; before the all-to-all the sequence
is split into R*U pieces in rank order; uneven splits give the first
(n mod parts) parts one extra element (as for Ring Anything's chunks).
"""

from __future__ import annotations

from typing import Dict, List

from .offsets import chunk_lengths


def _split(n: int, parts: int, uneven: bool) -> List[int]:
    """Sizes of `parts` consecutive pieces of n items."""
    return chunk_lengths(n, parts, ring_anything=uneven)


def cp_mesh(ring_degree: int, ulysses_degree: int) -> List[List[int]]:
    """mesh[r][u] = global rank at ring index r, Ulysses index u."""
    ranks = iter(range(ring_degree * ulysses_degree))
    return [[next(ranks) for _ in range(ulysses_degree)] for _ in range(ring_degree)]


def cp_share(seq_len: int, heads: int, ring_degree: int = 1, ulysses_degree: int = 1,
             ring_anything: bool = False, ulysses_anything: bool = False, rank: int = 0) -> Dict[str, int]:
    """The layout of `rank`: ring/Ulysses indices, its tokens before the
    all-to-all, and the query rows and heads of its attention share."""
    R, U = ring_degree, ulysses_degree
    if R < 1 or U < 1:
        raise ValueError("degrees must be >= 1")
    if ring_anything and ulysses_anything:
        raise ValueError("ring_anything and ulysses_anything do not combine")
    if ring_anything and not (R > 1 and U == 1):
        raise ValueError("ring_anything needs ring_degree > 1 and ulysses_degree 1")
    if ulysses_anything and not (U > 1 and R == 1):
        raise ValueError("ulysses_anything needs ulysses_degree > 1 and ring_degree 1")
    if heads < 1 or seq_len < 0:
        raise ValueError("bad sizes")
    if not (0 <= rank < R * U):
        raise ValueError("rank outside the grid")
    uneven = ring_anything or ulysses_anything
    if not uneven and heads % U != 0:
        raise ValueError(f"{heads} heads do not divide by ulysses_degree {U}")
    # sequence-parallel input: R*U pieces in rank order (raises when a plain
    # layout does not divide)
    piece_len = _split(seq_len, R * U, uneven)
    starts = [sum(piece_len[:g]) for g in range(R * U)]
    mesh = cp_mesh(R, U)
    r = next(i for i, row in enumerate(mesh) if rank in row)
    u = mesh[r].index(rank)
    # the Ulysses all-to-all gathers the pieces of the group (same r)
    group = mesh[r]
    rows = []
    for g in group:
        rows.extend(range(starts[g], starts[g] + piece_len[g]))
    assert rows == list(range(rows[0], rows[-1] + 1)) if rows else True
    head_len = _split(heads, U, uneven)
    h0 = sum(head_len[:u])
    return {
        "ring_index": r,
        "ulysses_index": u,
        "token_begin": starts[rank],
        "token_end": starts[rank] + piece_len[rank],
        "q_begin": rows[0] if rows else starts[group[0]],
        "q_end": rows[-1] + 1 if rows else starts[group[0]],
        "head_begin": h0,
        "head_end": h0 + head_len[u],
    }
