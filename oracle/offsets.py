"""Oracle side of the ring chunk partition (test infrastructure only).

Plain ring attention: the sequence length must divide evenly by the ring
degree (context-parallelism guide, "Paralelisme konteks", diffusers v0.43.0,
variant table: requirement of Ring Attention; the benchmark tables of the same
page report ring as failing at 1008x1008, where the length does not divide).

Ring Anything: any sequence length is accepted.  The local K/V blocks differ
in length; they travel in one buffer whose blocks all have the longest local
length, and only the true rows of each block take part in attention (same
guide, section "Ring Anything Attention"; Parallelism API page,
``ContextParallelConfig.ring_anything``).  The pages do not say which ranks
get the longer chunks; the reading taken here is that the first ``S mod N``
chunks hold one extra token, so lengths differ by at most one and the padded
length is ``ceil(S / N)``.
"""

from __future__ import annotations

from typing import List, Sequence


def chunk_lengths(seq_len: int, n_chunks: int, ring_anything: bool) -> List[int]:
    """Lengths of the N chunks of a length-``seq_len`` sequence, in ring order."""
    if not isinstance(seq_len, int) or not isinstance(n_chunks, int):
        raise TypeError("seq_len and n_chunks must be int")
    if n_chunks < 1:
        raise ValueError("n_chunks must be >= 1")
    if seq_len < 0:
        raise ValueError("seq_len must be >= 0")
    if not ring_anything and seq_len % n_chunks != 0:
        raise ValueError(
            f"plain ring attention needs seq_len divisible by the ring degree "
            f"({seq_len} % {n_chunks} = {seq_len % n_chunks}); use ring_anything"
        )
    lengths = []
    for i in range(n_chunks):
        # chunk i holds tokens [floor(i*S/N) ...] in the even case; in the
        # uneven case the first S mod N chunks are one token longer.
        base = seq_len // n_chunks
        extra = 1 if i < seq_len % n_chunks else 0
        lengths.append(base + extra)
    return lengths


def chunk_offsets(seq_len: int, n_chunks: int, ring_anything: bool = False) -> List[int]:
    """Offsets ``o[0..N]`` with ``o[0] = 0``, ``o[N] = seq_len``; chunk i is
    tokens ``[o[i], o[i+1])`` of the global sequence."""
    offsets = [0]
    for length in chunk_lengths(seq_len, n_chunks, ring_anything):
        offsets.append(offsets[-1] + length)
    return offsets


def padded_chunk_length(seq_len: int, n_chunks: int) -> int:
    """Length every rank pads its local K/V to before the all-gather: the
    longest local length over the ranks."""
    return max(chunk_lengths(seq_len, n_chunks, ring_anything=True))


def pad_gather_slice(local_blocks: Sequence[Sequence], pad_value=None) -> List[list]:
    """Simulate Ring Anything's exchange on plain Python lists.

    ``local_blocks[r]`` is rank r's local token list.  Each is padded to the
    longest local length with ``pad_value``, the padded blocks are stacked as
    an all-gather would deliver them, and each is cut back to its rank's true
    length.  Returns the list of recovered blocks (which must equal the input).
    """
    true_lengths = [len(b) for b in local_blocks]
    padded_len = max(true_lengths) if true_lengths else 0
    gathered = []
    for block in local_blocks:
        padded = list(block) + [pad_value] * (padded_len - len(block))
        gathered.append(padded)
    recovered = []
    for r, padded in enumerate(gathered):
        recovered.append(padded[: true_lengths[r]])
    return recovered
