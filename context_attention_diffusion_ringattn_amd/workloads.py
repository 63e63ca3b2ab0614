"""Seeded synthetic workloads for one GPU's share of ring attention.

This module only draws random inputs and names their shapes; it contains none
of the attention, partition or merge arithmetic.  The oracle and the HIP
library both consume what it produces (the same bf16-rounded tensors), and
neither is imported here.

Recipe (identical for every workload):

1. ``numpy.random.Generator(PCG64(seed))`` draws full-sequence float32
   standard normals ``[B, S, H, D]`` in the order Q, K, V -- one global tensor
   that every rank would slice its shard from, as the pages' example seeds one
   generator so that all ranks start from the same latents.
2. Outlier token rows (all heads and dims of a token) are then chosen with
   ``rng.choice(S, round(frac * S), replace=False)``, first for Q, then for K,
   and multiplied by the stated factor.
3. Everything is rounded to bfloat16 once (round to nearest even, via torch).
4. The local Q shard is rank 0's rows: the first ``q_rows`` tokens.

The pages measure FLUX.1-dev pipelines; these i.i.d. normal activations of
the same attention shapes stand in for them (no weights or prompts are used).
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    head_dim: int
    seq_len: int           # global sequence length S (K/V rows over all chunks)
    n_chunks: int          # ring degree N (1 for the Ulysses share)
    ring_anything: bool    # uneven split allowed
    q_rows: int            # local Q rows held by rank 0, as the workload states them
    seed: int
    fp32_inputs: bool = False      # drawn and consumed as fp32 by the oracle self-checks
    q_outlier_frac: float = 0.0
    q_outlier_scale: float = 1.0
    k_outlier_frac: float = 0.0
    k_outlier_scale: float = 1.0
    description: str = ""

    @property
    def flops(self) -> int:
        """Algorithmic flops of the shard: 4 * B * Sq * Skv * D * H (QK^T and PV)."""
        return 4 * self.batch * self.q_rows * self.seq_len * self.head_dim * self.heads


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(
        "tiny", batch=1, heads=2, head_dim=64, seq_len=256, n_chunks=2, ring_anything=False,
        q_rows=128, seed=0, fp32_inputs=True,
        description="B=1 H=2 D=64 S=256, ring degree 2 (chunks of 128), local Q = chunk 0, "
                    "fp32 N(0,1) inputs, scale 1/8"),
    "flux": Workload(
        "flux", batch=1, heads=24, head_dim=128, seq_len=4608, n_chunks=4, ring_anything=False,
        q_rows=1152, seed=1,
        description="Flux-like image DiT: B=1 H=24 D=128 S=4608 (4096 image + 512 text tokens), "
                    "ring degree 4, local Q 1152 rows vs 4 K/V chunks of 1152, bf16 N(0,1)"),
    "ring_anything": Workload(
        "ring_anything", batch=1, heads=24, head_dim=128, seq_len=4611, n_chunks=8, ring_anything=True,
        q_rows=577, seed=2, k_outlier_frac=0.01, k_outlier_scale=8.0,
        description="Ring Anything uneven split: B=1 H=24 D=128 S=4611 in 8 chunks (3 of 577, 5 of 576), "
                    "local Q = first chunk, bf16 N(0,1) with 1% of K rows x8"),
    "ulysses": Workload(
        "ulysses", batch=1, heads=6, head_dim=128, seq_len=16384, n_chunks=1, ring_anything=False,
        q_rows=16384, seed=3,
        description="Ulysses per-GPU share: B=1 S=16384, H=6 (24 heads / degree 4), D=128, "
                    "single full non-causal pass, bf16 N(0,1)"),
    "video": Workload(
        "video", batch=1, heads=24, head_dim=128, seq_len=65536, n_chunks=8, ring_anything=False,
        q_rows=8192, seed=4, q_outlier_frac=0.005, q_outlier_scale=6.0,
        k_outlier_frac=0.005, k_outlier_scale=6.0,
        description="Video-scale ring shard: B=1 H=24 D=128 S=65536 (16 frames x 64x64 tokens), "
                    "ring degree 8, local Q 8192 rows vs 8 K/V chunks of 8192, bf16 N(0,1) "
                    "with 0.5% Q/K outlier rows x6"),
    "usp": Workload(
        "usp", batch=1, heads=12, head_dim=128, seq_len=65536, n_chunks=4, ring_anything=False,
        q_rows=16384, seed=5,
        description="Unified (Ulysses 2 x ring 4, 8 GPUs) share of the video sequence: rank (r=0, u=0) "
                    "holds query rows 0..16383 (ring chunk 0) of heads 0..11 after the all-to-all and "
                    "attends to 4 K/V chunks of 16384, B=1 D=128, bf16 N(0,1)"),
    "ulysses_anything": Workload(
        "ulysses_anything", batch=1, heads=6, head_dim=128, seq_len=4481, n_chunks=1, ring_anything=False,
        q_rows=4481, seed=6,
        description="Ulysses Anything share of FLUX at 1008x1008 on 4 GPUs: S=4481 (3969 image + 512 text "
                    "tokens, not divisible by 4), 24 heads / 4 = 6 heads per GPU, one full non-causal "
                    "pass, B=1 D=128, bf16 N(0,1)"),
    "ring_even": Workload(
        "ring_even", batch=1, heads=24, head_dim=128, seq_len=4608, n_chunks=8, ring_anything=False,
        q_rows=576, seed=7, k_outlier_frac=0.01, k_outlier_scale=8.0,
        description="plain ring counterpart of ring_anything: B=1 H=24 D=128 S=4608 in 8 even chunks of "
                    "576, local Q = first chunk, bf16 N(0,1) with 1% of K rows x8"),
    "ulysses_even": Workload(
        "ulysses_even", batch=1, heads=6, head_dim=128, seq_len=4608, n_chunks=1, ring_anything=False,
        q_rows=4608, seed=8,
        description="plain Ulysses counterpart of ulysses_anything: FLUX at 1024x1024 on 4 GPUs, S=4608, "
                    "24 heads / 4 = 6 heads per GPU, one full non-causal pass, B=1 D=128, bf16 N(0,1)"),
}


def default_scale(head_dim: int) -> float:
    """The workloads' softmax scale 1/sqrt(D), as the float32 value the GPU is
    handed (returned as a Python float holding that exact value)."""
    return float(np.float32(1.0 / np.sqrt(np.float64(head_dim))))


def _draw(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def _outliers(rng: np.random.Generator, x: np.ndarray, frac: float, factor: float) -> np.ndarray:
    S = x.shape[1]
    count = int(round(frac * S))
    if count == 0:
        return np.zeros(0, dtype=np.int64)
    rows = rng.choice(S, count, replace=False)
    x[:, rows] *= np.float32(factor)
    return np.sort(rows)


def make_inputs(workload, *, seq_len: Optional[int] = None) -> dict:
    """Draw one workload's inputs.

    Returns a dict with

    * ``q_full``, ``k``, ``v``: bf16 CPU tensors ``[B, S, H, D]``;
    * ``q``: the local shard ``q_full[:, :q_rows]`` (a contiguous copy);
    * ``q_full_f32``, ``k_f32``, ``v_f32``: the float32 draws before bf16
      rounding (for the fp32 self-checks of the tiny workload);
    * ``scale``: the float32 softmax scale as a Python float;
    * ``q_outlier_rows``, ``k_outlier_rows``: the scaled token rows;
    * ``workload``: the ``Workload`` record.
    """
    w = WORKLOADS[workload] if isinstance(workload, str) else workload
    if seq_len is not None:
        w = dataclasses.replace(w, seq_len=seq_len)
    rng = np.random.Generator(np.random.PCG64(w.seed))
    shape = (w.batch, w.seq_len, w.heads, w.head_dim)
    q = _draw(rng, shape)
    k = _draw(rng, shape)
    v = _draw(rng, shape)
    q_rows_out = _outliers(rng, q, w.q_outlier_frac, w.q_outlier_scale)
    k_rows_out = _outliers(rng, k, w.k_outlier_frac, w.k_outlier_scale)
    q_full = torch.from_numpy(q).to(torch.bfloat16)
    k_b = torch.from_numpy(k).to(torch.bfloat16)
    v_b = torch.from_numpy(v).to(torch.bfloat16)
    return {
        "q_full": q_full,
        "k": k_b,
        "v": v_b,
        "q": q_full[:, : w.q_rows].contiguous(),
        "q_full_f32": q,
        "k_f32": k,
        "v_f32": v,
        "scale": default_scale(w.head_dim),
        "q_outlier_rows": q_rows_out,
        "k_outlier_rows": k_rows_out,
        "workload": w,
    }


def make_random(batch: int, q_len: int, kv_len: int, heads: int, head_dim: int, seed: int,
                k_outlier_frac: float = 0.0, k_outlier_scale: float = 1.0) -> dict:
    """Arbitrary-shape seeded inputs (bf16, N(0,1)) for parity cases that are
    not one of the named workloads.  Same recipe: Q, K, V drawn in that order,
    then K outlier rows."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _draw(rng, (batch, q_len, heads, head_dim))
    k = _draw(rng, (batch, kv_len, heads, head_dim))
    v = _draw(rng, (batch, kv_len, heads, head_dim))
    _outliers(rng, k, k_outlier_frac, k_outlier_scale)
    return {
        "q": torch.from_numpy(q).to(torch.bfloat16),
        "k": torch.from_numpy(k).to(torch.bfloat16),
        "v": torch.from_numpy(v).to(torch.bfloat16),
        "scale": default_scale(head_dim),
    }


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a (bf16 or fp32) CPU tensor, for the oracle."""
    return t.detach().to("cpu").to(torch.float64).numpy()
