"""Pins of the oracle's bf16-state ring (the convert_to_fp32 = False mode):
its bf16 rounding against the bit-level definition of round-to-nearest-even,
the one-chunk closed form, and exactness where no rounding can occur."""

import struct

import numpy as np

import oracle
from oracle.attention import _round_bf16


def _rne_bf16_by_definition(x: float) -> float:
    """float64 -> float32 (RNE, by struct) -> bf16 by rounding the float32 bit
    pattern to its upper 16 bits, ties to even; back to float."""
    if np.isinf(x):
        return x
    (bits,) = struct.unpack("<I", struct.pack("<f", x))
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFFFFFF
    (y,) = struct.unpack("<f", struct.pack("<I", bits & 0xFFFF0000))
    return y


def test_round_bf16_matches_definition():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(4000) * 10.0 ** rng.integers(-6, 6, size=4000),
        # exact ties between two bf16 neighbours: lower 16 bits of the float32 = 0x8000
        np.array([struct.unpack("<f", struct.pack("<I", (b << 16) | 0x8000))[0]
                  for b in rng.integers(0x0080, 0x7F00, size=500)], dtype=np.float64),
        np.array([-np.inf, 0.0, -0.0, 1.0, 3.0]),
    ])
    got = _round_bf16(vals)
    want = np.array([_rne_bf16_by_definition(float(v)) for v in vals])
    assert np.array_equal(got, want)


def test_one_chunk_is_the_rounded_definition():
    rng = np.random.default_rng(1)
    q, k, v = (rng.standard_normal((1, 9, 2, 8)), rng.standard_normal((1, 20, 2, 8)),
               rng.standard_normal((1, 20, 2, 8)))
    o, l = oracle.ring_shard_bf16_state_fp64(q, k, v, [0, 20], 0.4)
    eo, el = oracle.attention_fp64(q, k, v, 0.4)
    assert np.array_equal(o, _round_bf16(eo)) and np.array_equal(l, _round_bf16(el))


def test_constant_values_stay_exact():
    """With every value row equal to one bf16-representable vector, every
    partial and every merge of them is that vector, whatever the weights."""
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal((1, 7, 3, 8)), rng.standard_normal((1, 40, 3, 8))
    row = _round_bf16(rng.standard_normal(8) * 3.0)
    v = np.broadcast_to(row, (1, 40, 3, 8)).copy()
    o, _ = oracle.ring_shard_bf16_state_fp64(q, k, v, [0, 5, 17, 17, 40], 0.3)
    assert np.array_equal(o, np.broadcast_to(row, o.shape))


def test_bf16_state_error_exceeds_fp32_merge():
    """The float32 (here float64) merge reproduces one-shot attention; the
    bf16 state does not -- the effect the option exists to avoid."""
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((1, 16, 2, 16)), rng.standard_normal((1, 64, 2, 16)) * 2.0,
               rng.standard_normal((1, 64, 2, 16)))
    offs = [0, 8, 16, 24, 32, 40, 48, 56, 64]
    eo, el = oracle.attention_fp64(q, k, v, 0.25)
    ro, rl = oracle.ring_shard_fp64(q, k, v, offs, 0.25)
    bo, bl = oracle.ring_shard_bf16_state_fp64(q, k, v, offs, 0.25)
    assert np.max(np.abs(ro - eo)) < 1e-12 and np.max(np.abs(rl - el)) < 1e-12
    assert np.max(np.abs(bo - eo)) > 1e-4 and np.max(np.abs(bl - el)) > 1e-3
