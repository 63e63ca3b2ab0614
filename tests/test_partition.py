"""The context-parallel layout of a rank (ring x Ulysses grid): the oracle's
cp_share pinned to the pages' failure table, to partition properties that
any correct layout has, and to library routines; then the C ABI's
ringattn_cp_layout compared with it bit for bit (CPU only)."""

import ctypes
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
from context_attention_diffusion_ringattn_amd import _lib

CONFIGS = [
    # (S, H, R, U, ring_anything, ulysses_anything)
    (4608, 24, 1, 4, False, False), (4608, 24, 2, 2, False, False), (4608, 24, 4, 1, False, False),
    (65536, 24, 4, 2, False, False), (65536, 24, 8, 1, False, False), (16384, 24, 1, 4, False, False),
    (4611, 24, 8, 1, True, False), (4481, 24, 4, 1, True, False), (13, 3, 4, 1, True, False),
    (5, 2, 8, 1, True, False), (0, 4, 3, 1, True, False),
    (4481, 24, 1, 4, False, True), (4608, 24, 1, 5, False, True), (4481, 24, 1, 5, False, True),
    (7, 3, 1, 5, False, True), (100, 30, 1, 7, False, True), (0, 1, 1, 2, False, True),
    (48, 6, 3, 2, False, False), (96, 8, 2, 4, False, False), (12, 12, 1, 1, False, False),
]


def shares(S, H, R, U, ra, ua):
    return [oracle.cp_share(S, H, R, U, ra, ua, rank) for rank in range(R * U)]


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: "S{}H{}R{}U{}{}{}".format(*c[:4], "ra" * c[4], "ua" * c[5]))
def test_oracle_layout_is_a_partition(cfg):
    """Before the all-to-all the ranks' pieces tile [0, S) in rank order;
    after it the (query rows x heads) shares tile [0, S) x [0, H) exactly
    once; a Ulysses group's pieces make up its members' query rows; a ring
    group shares one head block and its query rows are the ring chunks."""
    S, H, R, U, ra, ua = cfg
    sh = shares(*cfg)
    pos = 0
    for s in sh:
        assert s["token_begin"] == pos and s["token_end"] >= pos
        pos = s["token_end"]
    assert pos == S
    cover = np.zeros((S, H), dtype=np.int64)
    for s in sh:
        cover[s["q_begin"]:s["q_end"], s["head_begin"]:s["head_end"]] += 1
    assert np.all(cover == 1)
    ring_chunks = oracle.chunk_offsets(S, R, ra)
    for s in sh:
        grp = [t for t in sh if t["ring_index"] == s["ring_index"]]
        assert len(grp) == U
        assert min(t["token_begin"] for t in grp) == s["q_begin"]
        assert max(t["token_end"] for t in grp) == s["q_end"]
        assert sum(t["token_end"] - t["token_begin"] for t in grp) == s["q_end"] - s["q_begin"]
        ring = [t for t in sh if t["ulysses_index"] == s["ulysses_index"]]
        assert len(ring) == R
        assert {(t["head_begin"], t["head_end"]) for t in ring} == {(s["head_begin"], s["head_end"])}
        assert [(t["q_begin"], t["q_end"]) for t in sorted(ring, key=lambda t: t["ring_index"])] == \
            list(zip(ring_chunks, ring_chunks[1:]))


def test_mesh_is_row_major_over_ring_then_ulysses():
    """A device mesh over dims ("ring", "ulysses") lays the ranks out as
    arange(world).reshape(R, U) (torch's mesh layout)."""
    for R, U in [(1, 4), (2, 2), (4, 2), (3, 5)]:
        assert oracle.cp_mesh(R, U) == torch.arange(R * U).reshape(R, U).tolist()
        for rank in range(R * U):
            s = oracle.cp_share(R * U * 6, 2 * U, R, U, False, False, rank)
            assert oracle.cp_mesh(R, U)[s["ring_index"]][s["ulysses_index"]] == rank


def test_uneven_splits_match_numpy_array_split():
    """Ulysses Anything: token pieces and head blocks are numpy.array_split's
    (the first n mod U parts one longer), e.g. 24 heads over 5 ranks."""
    for S, H, U in [(4481, 24, 4), (4608, 24, 5), (7, 3, 5), (100, 30, 7), (3, 2, 4)]:
        sh = shares(S, H, 1, U, False, True)
        assert [s["token_end"] - s["token_begin"] for s in sh] == [len(p) for p in np.array_split(np.arange(S), U)]
        assert [s["head_end"] - s["head_begin"] for s in sh] == [len(p) for p in np.array_split(np.arange(H), U)]
        assert all(s["q_begin"] == 0 and s["q_end"] == S for s in sh)
    assert [s["head_end"] - s["head_begin"] for s in shares(4608, 24, 1, 5, False, True)] == [5, 5, 5, 5, 4]


def test_reduces_to_ring_and_ulysses():
    """U = 1: the share is the ring chunk with all heads; R = 1: all rows with
    the Ulysses head range."""
    for S, R, ra in [(4608, 4, False), (4611, 8, True), (65536, 8, False)]:
        offs = oracle.chunk_offsets(S, R, ra)
        for r in range(R):
            s = oracle.cp_share(S, 24, R, 1, ra, False, r)
            assert (s["q_begin"], s["q_end"]) == (offs[r], offs[r + 1]) == (s["token_begin"], s["token_end"])
            assert (s["head_begin"], s["head_end"]) == (0, 24)
    for u in range(4):
        s = oracle.cp_share(16384, 24, 1, 4, False, False, u)
        assert (s["head_begin"], s["head_end"]) == oracle.ulysses_head_range(24, 4, u)
        assert (s["q_begin"], s["q_end"]) == (0, 16384)


def test_golden_variants_on_4_gpus(golden_dir):
    """The pages' 4-GPU FLUX tables: which variants run at 1024x1024 and at
    1008x1008."""
    with open(os.path.join(golden_dir, "flux_cp_variants_4gpu.json")) as f:
        fx = json.load(f)
    for c in fx["cases"]:
        args = (c["tokens"], fx["heads"], c["ring_degree"], c["ulysses_degree"], c["ring_anything"],
                c["ulysses_anything"])
        runs = True
        try:
            shares(*args)
        except ValueError:
            runs = False
        assert runs == (c["result"] == "runs"), c


def test_invalid_combinations():
    with pytest.raises(ValueError):
        oracle.cp_share(16, 4, 2, 2, True, False, 0)     # ring_anything with Ulysses
    with pytest.raises(ValueError):
        oracle.cp_share(16, 4, 2, 2, False, True, 0)     # ulysses_anything with a ring
    with pytest.raises(ValueError):
        oracle.cp_share(16, 4, 2, 1, True, True, 0)
    with pytest.raises(ValueError):
        oracle.cp_share(16, 6, 1, 4, False, False, 0)    # heads do not divide
    with pytest.raises(ValueError):
        oracle.cp_share(16, 4, 2, 2, False, False, 4)    # rank outside the grid


# ---------------------------------------------------------------- C ABI ----

@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def c_share(L, S, H, R, U, ra, ua, rank):
    cfg = _lib.CpConfig(seq_len=S, heads=H, ring_degree=R, ulysses_degree=U, ring_anything=int(ra),
                        ulysses_anything=int(ua), reserved=0)
    out = _lib.CpShare()
    st = L.ringattn_cp_layout(ctypes.byref(cfg), rank, ctypes.byref(out))
    return st, {k: getattr(out, k) for k, _ in _lib.CpShare._fields_}


def test_c_share_bit_exact_vs_oracle(L):
    """Every rank of a sweep of grids, plain and uneven, valid and invalid."""
    cases = list(CONFIGS)
    for S, H, R, U in itertools.product([0, 1, 7, 48, 4481, 4608], [1, 5, 24], [1, 2, 3, 8], [1, 2, 4, 5]):
        for ra, ua in [(False, False), (True, False), (False, True)]:
            cases.append((S, H, R, U, ra, ua))
    n_ok = n_err = 0
    for S, H, R, U, ra, ua in cases:
        for rank in range(-1, R * U + 1):
            st, got = c_share(L, S, H, R, U, ra, ua, rank)
            try:
                want = oracle.cp_share(S, H, R, U, ra, ua, rank)
            except ValueError:
                assert st == _lib.RINGATTN_EINVAL, (S, H, R, U, ra, ua, rank, got)
                n_err += 1
                continue
            assert st == 0, (S, H, R, U, ra, ua, rank, _lib.last_error())
            assert got == want, (S, H, R, U, ra, ua, rank)
            n_ok += 1
    print(f"{n_ok} valid and {n_err} invalid (config, rank) pairs compared")
    assert n_ok > 500 and n_err > 500


def test_c_share_argument_errors(L):
    cfg = _lib.CpConfig(seq_len=16, heads=4, ring_degree=2, ulysses_degree=2, ring_anything=0, ulysses_anything=0,
                        reserved=1)
    out = _lib.CpShare()
    assert L.ringattn_cp_layout(ctypes.byref(cfg), 0, ctypes.byref(out)) == _lib.RINGATTN_EINVAL
    cfg.reserved = 0
    assert L.ringattn_cp_layout(None, 0, ctypes.byref(out)) == _lib.RINGATTN_EINVAL
    assert L.ringattn_cp_layout(ctypes.byref(cfg), 0, None) == _lib.RINGATTN_EINVAL
    cfg.ring_degree = 129
    assert L.ringattn_cp_layout(ctypes.byref(cfg), 0, ctypes.byref(out)) == _lib.RINGATTN_EINVAL


# ------------------------------------------------------------ mutants ----

from oracle.partition import cp_share as _true_share


def _mutant(kind):
    """cp_share as a plausible mistaken implementation would return it."""
    def f(S, H, R, U, ra, ua, rank):
        good = _true_share(S, H, R, U, ra, ua, rank)
        if kind == "column_major_mesh":      # rank = u * R + r
            other = _true_share(S, H, R, U, ra, ua, (rank % R) * U + rank // R)
            return dict(other, token_begin=good["token_begin"], token_end=good["token_end"])
        if kind == "heads_extra_to_last":
            n = [len(p) for p in np.array_split(np.arange(H), U)][::-1]
            h0 = sum(n[:good["ulysses_index"]])
            return dict(good, head_begin=h0, head_end=h0 + n[good["ulysses_index"]])
        if kind == "no_all_to_all_gather":   # query rows = the rank's own piece
            return dict(good, q_begin=good["token_begin"], q_end=good["token_end"])
        raise AssertionError(kind)
    return f


@pytest.mark.parametrize("kind", ["column_major_mesh", "heads_extra_to_last", "no_all_to_all_gather"])
def test_partition_mutants_caught(kind, monkeypatch):
    """Each mutant fails at least one of the pins above."""
    monkeypatch.setattr(oracle, "cp_share", _mutant(kind))
    caught = False
    checks = [lambda: test_mesh_is_row_major_over_ring_then_ulysses(),
              lambda: test_uneven_splits_match_numpy_array_split()]
    checks += [lambda c=c: test_oracle_layout_is_a_partition(c) for c in CONFIGS]
    for chk in checks:
        try:
            chk()
        except AssertionError:
            caught = True
            break
    assert caught, f"mutant {kind} passed every partition pin"
