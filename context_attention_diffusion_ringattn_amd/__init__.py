"""MI355X-native (gfx950) ring-attention shard: one GPU's share of context
parallel attention -- a local Q shard attending to N K/V chunks with a float32
log-sum-exp merge, the uneven Ring Anything split and the Ulysses head share.

The compute lives in the HIP library ``libringattn.so`` (C ABI in
``include/ringattn.h``); this package is a thin torch-tensor binding over it.
"""

from .ringattn import (
    RingConfig,
    acc_init,
    chunk_offsets,
    cp_share,
    default_scale,
    forward,
    forward_plan,
    merge,
    new_accumulators,
    new_accumulators_bf16,
    new_workspace,
    step_plan,
    ring_shard,
    ring_sweep,
    step,
    step_bf16,
)
from ._lib import RingAttnError

__all__ = [
    "RingConfig",
    "RingAttnError",
    "acc_init",
    "chunk_offsets",
    "cp_share",
    "default_scale",
    "forward",
    "forward_plan",
    "merge",
    "new_accumulators",
    "new_accumulators_bf16",
    "new_workspace",
    "step_plan",
    "ring_shard",
    "ring_sweep",
    "step",
    "step_bf16",
]
