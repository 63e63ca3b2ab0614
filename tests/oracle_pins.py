"""Pins for the oracle: checks against facts other than the oracle itself.

Each check takes the implementation under test as arguments so the same
checks run on the real oracle (``test_oracle.py``) and on deliberately broken
copies of it (``test_oracle_mutants.py``), which must each fail at least one
check.  Nothing here retypes the oracle's formula: the references are a
library routine (torch's SDPA and logsumexp in float64), brute force with
``math.fsum``, closed forms and invariants of softmax attention.
"""

from __future__ import annotations

import itertools
import math

import numpy as np
import torch

from oracle import brute_force_attention, chunk_offsets


def rand(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape) * scale


def check_matches_torch_sdpa(attn, shapes=((1, 7, 2, 8, 11), (2, 33, 3, 16, 50), (1, 128, 2, 64, 256)),
                             scale=None, tol=1e-12):
    """ring_degree = 1 is plain attention: compare with torch's float64 SDPA
    (output) and logsumexp (LSE), both library routines."""
    for n, (B, Sq, H, D, Skv) in enumerate(shapes):
        q = rand((B, Sq, H, D), 10 + n)
        k = rand((B, Skv, H, D), 20 + n)
        v = rand((B, Skv, H, D), 30 + n)
        sc = 1.0 / math.sqrt(D) if scale is None else scale
        out, lse = attn(q, k, v, sc)
        qt = torch.from_numpy(q).permute(0, 2, 1, 3)
        kt = torch.from_numpy(k).permute(0, 2, 1, 3)
        vt = torch.from_numpy(v).permute(0, 2, 1, 3)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=sc)
        ref = ref.permute(0, 2, 1, 3).numpy()
        ref_lse = torch.logsumexp(sc * torch.matmul(qt, kt.transpose(-1, -2)), dim=-1).numpy()
        assert np.max(np.abs(out - ref)) <= tol, "output differs from torch SDPA"
        assert np.max(np.abs(lse - ref_lse)) <= tol, "LSE differs from torch logsumexp"


def check_brute_force(attn, cases=((1, 3, 1, 2, 4), (2, 5, 2, 3, 7), (1, 4, 3, 8, 16), (1, 1, 1, 1, 1)),
                      tol=1e-13):
    """Agreement with pure-Python loops on tiny shapes."""
    for n, (B, Sq, H, D, Skv) in enumerate(cases):
        q = rand((B, Sq, H, D), 100 + n, 1.5)
        k = rand((B, Skv, H, D), 200 + n, 1.5)
        v = rand((B, Skv, H, D), 300 + n)
        sc = 0.37 + 0.1 * n
        out, lse = attn(q, k, v, sc)
        bo, bl = brute_force_attention(q.tolist(), k.tolist(), v.tolist(), sc)
        assert np.max(np.abs(out - np.array(bo))) <= tol, "output differs from brute force"
        assert np.max(np.abs(lse - np.array(bl))) <= tol, "LSE differs from brute force"


def check_constant_v(attn, tol=1e-14):
    """If every value row is the same vector c, every output row is c."""
    B, Sq, H, D, Skv = 1, 9, 2, 16, 40
    q = rand((B, Sq, H, D), 1, 3.0)
    k = rand((B, Skv, H, D), 2, 3.0)
    c = rand((B, 1, H, D), 3)
    v = np.broadcast_to(c, (B, Skv, H, D)).copy()
    out, _ = attn(q, k, v, 0.25)
    assert np.max(np.abs(out - np.broadcast_to(c, out.shape))) <= tol, "constant V not returned"


def check_zero_keys(attn, tol=1e-13):
    """With K = 0 every score is 0: out is the mean of the V rows and
    lse = ln(Skv) (closed form)."""
    B, Sq, H, D, Skv = 1, 5, 3, 8, 37
    q = rand((B, Sq, H, D), 4)
    k = np.zeros((B, Skv, H, D))
    v = rand((B, Skv, H, D), 5)
    out, lse = attn(q, k, v, 0.5)
    mean = v.mean(axis=1, keepdims=True)
    assert np.max(np.abs(out - np.broadcast_to(mean, out.shape))) <= tol, "K=0: out != mean(V)"
    assert np.max(np.abs(lse - math.log(Skv))) <= tol, "K=0: lse != ln Skv"


def check_closed_form_two_keys(attn, tol=1e-15):
    """One query, two keys, scale 1: q = (1, 0), k1 = (1, 0), k2 = (0, 0),
    v1 = (1, 0), v2 = (0, 1).  Scores are (1, 0), so lse = ln(1 + e) and
    out = (e, 1) / (1 + e).  Also: scale 2 with k1 = (0, 3) gives scores
    (0, 0) -> lse = ln 2, out = (0.5, 0.5)."""
    q = np.array([1.0, 0.0]).reshape(1, 1, 1, 2)
    k = np.array([[1.0, 0.0], [0.0, 0.0]]).reshape(1, 2, 1, 2)
    v = np.array([[1.0, 0.0], [0.0, 1.0]]).reshape(1, 2, 1, 2)
    out, lse = attn(q, k, v, 1.0)
    e = math.e
    assert abs(lse[0, 0, 0] - math.log(1.0 + e)) <= tol, "two-key lse"
    assert abs(out[0, 0, 0, 0] - e / (1.0 + e)) <= tol and abs(out[0, 0, 0, 1] - 1.0 / (1.0 + e)) <= tol, \
        "two-key out"
    k2 = np.array([[0.0, 3.0], [0.0, 0.0]]).reshape(1, 2, 1, 2)
    out, lse = attn(q, k2, v, 2.0)
    assert abs(lse[0, 0, 0] - math.log(2.0)) <= tol and np.max(np.abs(out[0, 0, 0] - 0.5)) <= tol, \
        "tied scores"


def check_score_shift(attn, tol=1e-12):
    """Adding a vector u to every key adds scale * (q_i . u) to every score of
    row i: out is unchanged and lse shifts by exactly that amount."""
    B, Sq, H, D, Skv = 1, 6, 2, 8, 21
    q = rand((B, Sq, H, D), 6)
    k = rand((B, Skv, H, D), 7)
    v = rand((B, Skv, H, D), 8)
    u = rand((B, 1, H, D), 9)
    sc = 0.7
    out1, lse1 = attn(q, k, v, sc)
    out2, lse2 = attn(q, k + u, v, sc)
    shift = sc * np.einsum("bshd,bhd->bhs", q, u[:, 0])
    assert np.max(np.abs(out1 - out2)) <= tol, "key shift changed out"
    assert np.max(np.abs(lse2 - lse1 - shift)) <= tol, "key shift: lse did not move by scale*q.u"


def check_head_independence(attn, tol=0.0):
    """Ulysses share: computing all heads and keeping heads [lo, hi) equals
    computing only those heads (heads never mix)."""
    B, S, H, D = 1, 24, 8, 8
    q = rand((B, S, H, D), 11)
    k = rand((B, S, H, D), 12)
    v = rand((B, S, H, D), 13)
    full_out, full_lse = attn(q, k, v, 0.3)
    for lo, hi in ((0, 2), (2, 4), (6, 8)):
        out, lse = attn(q[:, :, lo:hi], k[:, :, lo:hi], v[:, :, lo:hi], 0.3)
        assert np.max(np.abs(out - full_out[:, :, lo:hi])) <= tol, "head slice out"
        assert np.max(np.abs(lse - full_lse[:, lo:hi])) <= tol, "head slice lse"


def check_merge_equals_one_shot(attn, merge, ring, tol=1e-12):
    """Folding every chunk partial with the merge gives one-shot attention over
    the whole sequence; even chunks, ragged chunks and empty chunks."""
    cases = [
        ((1, 16, 2, 8), 64, chunk_offsets(64, 4)),
        ((2, 5, 3, 4), 13, chunk_offsets(13, 4, ring_anything=True)),
        ((1, 7, 1, 16), 3, chunk_offsets(3, 5, ring_anything=True)),   # two empty chunks
        ((1, 9, 2, 8), 50, [0, 1, 1, 30, 49, 50]),
    ]
    for n, ((B, Sq, H, D), S, offs) in enumerate(cases):
        q = rand((B, Sq, H, D), 40 + n, 1.2)
        k = rand((B, S, H, D), 50 + n, 1.2)
        v = rand((B, S, H, D), 60 + n)
        out, lse = attn(q, k, v, 0.45)
        rout, rlse = ring(q, k, v, offs, 0.45)
        assert np.max(np.abs(out - rout)) <= tol, "merged out != one-shot"
        assert np.max(np.abs(lse - rlse)) <= tol, "merged lse != one-shot"


def check_merge_order_invariance(attn, merge, ring, tol=1e-12):
    """The merge result does not depend on the order the chunks arrive in:
    every order for N <= 4, 20 random orders for N = 8."""
    B, Sq, H, D = 1, 6, 2, 8
    for N, S in ((2, 10), (3, 17), (4, 23), (8, 61)):
        q = rand((B, Sq, H, D), 70 + N)
        k = rand((B, S, H, D), 80 + N, 1.5)
        v = rand((B, S, H, D), 90 + N)
        offs = chunk_offsets(S, N, ring_anything=True)
        ref_out, ref_lse = ring(q, k, v, offs, 0.6)
        if N <= 4:
            orders = list(itertools.permutations(range(N)))
        else:
            rng = np.random.default_rng(N)
            orders = [tuple(rng.permutation(N)) for _ in range(20)]
        for order in orders:
            out, lse = ring(q, k, v, offs, 0.6, order=order)
            assert np.max(np.abs(out - ref_out)) <= tol and np.max(np.abs(lse - ref_lse)) <= tol, \
                f"order {order} changed the result"


def check_self_merge(attn, merge, tol=1e-14):
    """Merging a partial with itself leaves out unchanged and adds ln 2 to lse."""
    B, Sq, H, D, S = 1, 8, 2, 8, 19
    out, lse = attn(rand((B, Sq, H, D), 21), rand((B, S, H, D), 22), rand((B, S, H, D), 23), 0.5)
    mo, ml = merge(out, lse, out, lse)
    assert np.max(np.abs(mo - out)) <= tol, "self-merge changed out"
    assert np.max(np.abs(ml - lse - math.log(2.0))) <= tol, "self-merge lse != lse + ln 2"


def check_empty_partial_identity(attn, merge):
    """A partial with lse = -inf is the merge identity, on either side, even
    when its output holds NaN/inf garbage; two empties stay empty."""
    B, Sq, H, D, S = 1, 4, 2, 8, 9
    out, lse = attn(rand((B, Sq, H, D), 31), rand((B, S, H, D), 32), rand((B, S, H, D), 33), 0.5)
    garbage = np.full_like(out, np.nan)
    garbage[..., 0] = np.inf
    empty_lse = np.full_like(lse, -np.inf)
    for mo, ml in (merge(out, lse, garbage, empty_lse), merge(garbage, empty_lse, out, lse)):
        assert np.array_equal(mo, out) and np.array_equal(ml, lse), "empty partial is not the identity"
    mo, ml = merge(garbage, empty_lse, garbage, empty_lse)
    assert np.all(ml == -np.inf) and not np.any(np.isnan(mo)), "two empties must stay (0, -inf)"


def check_merge_associativity(attn, merge, tol=1e-13):
    """(a + b) + c == a + (b + c) for the merge."""
    B, Sq, H, D = 1, 5, 2, 8
    q = rand((B, Sq, H, D), 41)
    parts = []
    for n, S in enumerate((7, 12, 3)):
        parts.append(attn(q, rand((B, S, H, D), 42 + n, 2.0), rand((B, S, H, D), 45 + n), 0.8))
    (ao, al), (bo, bl), (co, cl) = parts
    lo, ll = merge(*merge(ao, al, bo, bl), co, cl)
    ro, rl = merge(ao, al, *merge(bo, bl, co, cl))
    assert np.max(np.abs(lo - ro)) <= tol and np.max(np.abs(ll - rl)) <= tol, "merge not associative"


ATTENTION_CHECKS = [
    check_matches_torch_sdpa,
    check_brute_force,
    check_constant_v,
    check_zero_keys,
    check_closed_form_two_keys,
    check_score_shift,
    check_head_independence,
]

MERGE_CHECKS = [
    check_merge_equals_one_shot,
    check_merge_order_invariance,
]

MERGE_ONLY_CHECKS = [
    check_self_merge,
    check_empty_partial_identity,
    check_merge_associativity,
]
