"""Planted mistakes in copies of the oracle, on the CPU: every mutant must be
caught by at least one pin.  This shows the pins are strong enough that a
plausible slip (a dropped term, a wrong sign or index, a transposed operand)
in the oracle could not go unnoticed."""

import math

import numpy as np
import pytest

from oracle import attention_fp64, lse_merge_fp64, ring_shard_fp64
from oracle_pins import ATTENTION_CHECKS, MERGE_CHECKS, MERGE_ONLY_CHECKS


def _attn_generic(q, k, v, scale, *, drop_scale=False, no_max=False, lse_drop_max=False,
                  transpose_v_heads=False, sum_over_d_wrong=False, exp_sign=1.0, use_mean=False):
    q = np.asarray(q, float)
    k = np.asarray(k, float)
    v = np.asarray(v, float)
    B, Sq, H, D = q.shape
    Skv = k.shape[1]
    out = np.zeros((B, Sq, H, D))
    lse = np.full((B, H, Sq), -np.inf)
    if Skv == 0:
        return out, lse
    for b in range(B):
        for h in range(H):
            hv = (H - 1 - h) if transpose_v_heads else h
            s = (q[b, :, h] @ k[b, :, h].T) * (1.0 if drop_scale else scale)
            if sum_over_d_wrong:
                s = s + scale * q[b, :, h].sum(axis=1, keepdims=True)
            m = np.zeros(Sq) if no_max else s.max(axis=1)
            l = np.exp(exp_sign * (s - m[:, None])).sum(axis=1)
            row_lse = (0.0 if lse_drop_max else m) + np.log(l)
            w = np.exp(exp_sign * (s - m[:, None])) / l[:, None]
            if use_mean:
                w = np.full_like(w, 1.0 / Skv)
            out[b, :, h] = w @ v[b, :, hv]
            lse[b, h] = row_lse
    return out, lse


ATTENTION_MUTANTS = {
    "drop_scale": dict(drop_scale=True),
    "lse_without_max": dict(lse_drop_max=True),
    "v_from_wrong_head": dict(transpose_v_heads=True),
    "extra_score_term": dict(sum_over_d_wrong=True),
    "exp_sign_flipped": dict(exp_sign=-1.0),
    "uniform_weights": dict(use_mean=True),
}


@pytest.mark.parametrize("name", sorted(ATTENTION_MUTANTS))
def test_attention_mutant_caught(name):
    kw = ATTENTION_MUTANTS[name]

    def mutant(q, k, v, scale):
        return _attn_generic(q, k, v, scale, **kw)

    caught = []
    for check in ATTENTION_CHECKS:
        try:
            check(mutant)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"mutant {name} passed every attention pin"


def _merge_mutant(kind):
    def merge(out_a, lse_a, out_b, lse_b):
        out_a = np.asarray(out_a, float)
        out_b = np.asarray(out_b, float)
        lse_a = np.asarray(lse_a, float)
        lse_b = np.asarray(lse_b, float)
        B, H, Sq = lse_a.shape
        out = np.zeros_like(out_a)
        lse = np.full_like(lse_a, -np.inf)
        for b in range(B):
            for h in range(H):
                for i in range(Sq):
                    a, c = lse_a[b, h, i], lse_b[b, h, i]
                    if a == -np.inf and c == -np.inf:
                        continue
                    if kind != "multiply_empty" and a == -np.inf:
                        out[b, i, h], lse[b, h, i] = out_b[b, i, h], c
                        continue
                    if kind != "multiply_empty" and c == -np.inf:
                        out[b, i, h], lse[b, h, i] = out_a[b, i, h], a
                        continue
                    m = max(a, c)
                    if kind == "wrong_sign":
                        new = m + math.log1p(math.exp(abs(a - c)))
                    elif kind == "plain_average":
                        new = m + math.log1p(math.exp(-abs(a - c)))
                    elif kind == "max_only":
                        new = m
                    else:
                        new = m + math.log1p(math.exp(-abs(a - c)))
                    if kind == "plain_average":
                        o = 0.5 * (out_a[b, i, h] + out_b[b, i, h])
                    elif kind == "swapped_weights":
                        o = math.exp(c - new) * out_a[b, i, h] + math.exp(a - new) * out_b[b, i, h]
                    else:
                        o = math.exp(a - new) * out_a[b, i, h] + math.exp(c - new) * out_b[b, i, h]
                    out[b, i, h], lse[b, h, i] = o, new
        return out, lse
    return merge


MERGE_MUTANTS = ["wrong_sign", "plain_average", "max_only", "swapped_weights", "multiply_empty"]


@pytest.mark.parametrize("kind", MERGE_MUTANTS)
def test_merge_mutant_caught(kind):
    merge = _merge_mutant(kind)

    def ring(q, k, v, offsets, scale, order=None):
        q = np.asarray(q, float)
        n = len(offsets) - 1
        B, Sq, H, D = q.shape
        out = np.zeros((B, Sq, H, D))
        lse = np.full((B, H, Sq), -np.inf)
        for c in (range(n) if order is None else order):
            po, pl = attention_fp64(q, np.asarray(k)[:, offsets[c]:offsets[c + 1]],
                                    np.asarray(v)[:, offsets[c]:offsets[c + 1]], scale)
            with np.errstate(invalid="ignore", over="ignore"):
                out, lse = merge(out, lse, po, pl)
        return out, lse

    caught = []
    for check in MERGE_CHECKS:
        try:
            check(attention_fp64, merge, ring)
        except AssertionError:
            caught.append(check.__name__)
    for check in MERGE_ONLY_CHECKS:
        try:
            with np.errstate(invalid="ignore", over="ignore"):
                check(attention_fp64, merge)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"merge mutant {kind} passed every merge pin"


def test_real_oracle_passes_everything():
    for check in ATTENTION_CHECKS:
        check(attention_fp64)
    for check in MERGE_CHECKS:
        check(attention_fp64, lse_merge_fp64, ring_shard_fp64)
    for check in MERGE_ONLY_CHECKS:
        check(attention_fp64, lse_merge_fp64)


# ------------------------------------------------------------- offsets ----

def _lengths_mutant(kind):
    def lengths(S, N, ring_anything=True):
        if kind == "no_divisibility_check":
            pass
        elif not ring_anything and S % N:
            raise ValueError("not divisible")
        base, rem = divmod(S, N)
        if kind == "extra_to_last":
            return [base + (1 if i >= N - rem else 0) for i in range(N)]
        if kind == "off_by_one_remainder":
            return [base + (1 if i < rem + 1 else 0) for i in range(N)]
        if kind == "remainder_on_last":
            return [base] * (N - 1) + [base + rem]
        if kind == "ceil_then_rest":
            c = -(-S // N)
            out, left = [], S
            for _ in range(N):
                out.append(min(c, left))
                left -= out[-1]
            return out
        return [base + (1 if i < rem else 0) for i in range(N)]
    return lengths


OFFSET_MUTANTS = ["extra_to_last", "off_by_one_remainder", "remainder_on_last", "ceil_then_rest",
                  "no_divisibility_check"]


def _offset_pins_catch(lengths):
    """The offset pins of test_oracle.py, applied to a candidate lengths rule:
    numpy.array_split, the 577/576 split of S=4611 over 8, and the pages'
    divisibility failure at 1008x1008 on 4 GPUs."""
    for S in range(0, 120):
        for N in range(1, 11):
            if lengths(S, N) != [len(p) for p in np.array_split(np.arange(S), N)]:
                return True
    if lengths(4611, 8) != [577] * 3 + [576] * 5:
        return True
    try:
        lengths(4481, 4, ring_anything=False)
    except ValueError:
        return False
    return True


@pytest.mark.parametrize("kind", OFFSET_MUTANTS)
def test_offsets_mutant_caught(kind):
    assert _offset_pins_catch(_lengths_mutant(kind)), f"offsets mutant {kind} passed every offset pin"


def test_offset_pins_accept_the_oracle():
    from oracle import chunk_lengths
    assert not _offset_pins_catch(lambda S, N, ring_anything=True: chunk_lengths(S, N, ring_anything))
