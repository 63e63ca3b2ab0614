"""GPU parity of the whole ring on one GPU (``ringattn_ring_sweep``): every
rank's shard, each visiting the chunks in its rank-rotated order with a
float32 merge after every step, reassembled and compared with the oracle's
one-shot attention of every query row over all S keys.

Tolerances as for the single shard: max |out - oracle| <= 1e-2,
max |lse - oracle| <= 1e-3.  Small cases are compared in full; the Flux-like,
Ring Anything and video rings on sampled rows of every rank (first and last
row of each rank included), which the oracle computes one by one.
"""

import functools

import numpy as np
import pytest
import torch

import oracle
from context_attention_diffusion_ringattn_amd import workloads as W

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2
LSE_TOL = 1e-3


@pytest.fixture(scope="module")
def ra():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    import context_attention_diffusion_ringattn_amd as ra_mod
    ra_mod._lib.lib()
    return ra_mod


def dev(t):
    return t.to("cuda:0")


def assert_close(gpu_out, gpu_lse, ref_out, ref_lse, what):
    o = gpu_out.detach().to("cpu", torch.float64).numpy()
    l = gpu_lse.detach().to("cpu", torch.float64).numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), f"{what}: non-finite GPU result"
    eo = float(np.max(np.abs(o - ref_out)))
    el = float(np.max(np.abs(l - ref_lse)))
    print(f"{what}: max|dout|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= OUT_TOL, f"{what}: out error {eo}"
    assert el <= LSE_TOL, f"{what}: lse error {el}"


def rank_rows(offs, per_rank, seed):
    """First and last row of every non-empty rank plus `per_rank` random rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    for r in range(len(offs) - 1):
        lo, hi = offs[r], offs[r + 1]
        if hi == lo:
            continue
        rows.update([lo, hi - 1])
        rows.update(int(x) for x in rng.integers(lo, hi, size=min(per_rank, hi - lo)))
    return sorted(rows)


def padded(x, offs, fill):
    """Ring Anything's padded all-gather buffer of k or v: chunk c at rows
    c * pad, pad = the longest chunk, padding rows set to `fill`."""
    lens = [b - a for a, b in zip(offs, offs[1:])]
    pad = max(max(lens), 1)
    B, _, H, D = x.shape
    xp = torch.full((B, len(lens) * pad, H, D), fill, dtype=x.dtype)
    for c, n in enumerate(lens):
        xp[:, c * pad:c * pad + n] = x[:, offs[c]:offs[c + 1]]
    return xp, pad


@functools.lru_cache(maxsize=None)
def workload_inputs(name):
    return W.make_inputs(name)


SMALL_CASES = [
    # (B, H, D, S, ring degree, ring_anything, seed)
    (1, 2, 64, 256, 2, False, 0),        # the tiny workload's shape
    (2, 3, 64, 300, 7, True, 200),       # 6 ranks of 43 rows, 1 of 42
    (1, 2, 128, 5, 8, True, 201),        # 3 empty ranks / chunks
    (1, 1, 128, 1000, 3, True, 202),     # 334, 333, 333: ragged tails
    (3, 2, 128, 520, 4, False, 203),     # 4 x 130
    (1, 2, 64, 203, 40, True, 204),      # 40 ranks: above the batched-launch limit (per-rank launches)
    (1, 3, 128, 161, 32, True, 205),     # 32 ranks: the largest batched ring step
]


@pytest.mark.parametrize("case", SMALL_CASES, ids=lambda c: f"B{c[0]}H{c[1]}D{c[2]}S{c[3]}N{c[4]}")
def test_sweep_small_full(ra, case):
    B, H, D, S, N, anything, seed = case
    print(f"case sweep {case}", flush=True)
    x = W.make_random(B, S, S, H, D, seed, k_outlier_frac=0.05, k_outlier_scale=5.0)
    offs = ra.chunk_offsets(S, N, anything)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    ref_out, ref_lse = oracle.attention_fp64(W.to_f64(x["q"]), W.to_f64(x["k"]), W.to_f64(x["v"]), x["scale"])
    out, lse = ra.ring_sweep(q, k, v, chunk_offsets=offs, scale=x["scale"])
    torch.cuda.synchronize()
    assert_close(out, lse, ref_out, ref_lse, "sweep packed")
    kp, pad = padded(x["k"], offs, float("nan"))
    vp, _ = padded(x["v"], offs, float("nan"))
    out2, lse2 = ra.ring_sweep(q, dev(kp), dev(vp), chunk_offsets=offs, kv_chunk_stride=pad, scale=x["scale"])
    torch.cuda.synchronize()
    assert_close(out2, lse2, ref_out, ref_lse, "sweep padded")


def test_sweep_rank_equals_its_shard(ra):
    """Each rank's rows of the sweep equal that rank's own shard computed alone
    (forward over the packed chunks in all-gather order) up to rounding, and
    the step path in the same rotated order, with the sweep's workgroup shape
    (256 query rows, one split), gives the same bits as the sweep."""
    x = workload_inputs("ring_anything")
    w = x["workload"]
    offs = ra.chunk_offsets(w.seq_len, w.n_chunks, True)
    qf, k, v = dev(x["q_full"]), dev(x["k"]), dev(x["v"])
    out, lse = ra.ring_sweep(qf, k, v, chunk_offsets=offs, scale=x["scale"])
    for r in (0, 3, 7):
        lo, hi = offs[r], offs[r + 1]
        q_r = qf[:, lo:hi].contiguous()
        o_f, l_f = ra.forward(q_r, k, v, chunk_offsets=offs, scale=x["scale"])
        o_s, l_s = ra.new_accumulators(q_r)
        for s in range(w.n_chunks):
            c = (r + s) % w.n_chunks
            ra.step(q_r, k[:, offs[c]:offs[c + 1]].contiguous(), v[:, offs[c]:offs[c + 1]].contiguous(), o_s, l_s,
                    scale=x["scale"], n_splits=1, block_m=256)
        torch.cuda.synchronize()
        assert torch.equal(o_s, out[:, lo:hi]) and torch.equal(l_s, lse[:, :, lo:hi]), f"rank {r}"
        d_out = (o_f - out[:, lo:hi]).abs().max().item()
        d_lse = (l_f - lse[:, :, lo:hi]).abs().max().item()
        print(f"rank {r}: |sweep - forward| out {d_out:.2e} lse {d_lse:.2e}", flush=True)
        assert d_out <= OUT_TOL and d_lse <= LSE_TOL


@pytest.mark.parametrize("name", ["flux", "ring_anything", "video"])
def test_sweep_workloads_sampled(ra, name):
    """The full rings of the Flux-like (4 ranks), Ring Anything (8 ranks of
    577 / 576 rows) and video (8 ranks of 8192) workloads, with the packed
    buffer and, for Ring Anything, the padded one; sampled rows of every rank."""
    x = workload_inputs(name)
    w = x["workload"]
    print(f"case sweep {name}: S={w.seq_len} N={w.n_chunks}", flush=True)
    offs = ra.chunk_offsets(w.seq_len, w.n_chunks, w.ring_anything)
    qf, k, v = dev(x["q_full"]), dev(x["k"]), dev(x["v"])
    rows = rank_rows(offs, 2 if name == "video" else 6, w.seed)
    ref_out, ref_lse = oracle.attention_rows_fp64(W.to_f64(x["q_full"]), W.to_f64(x["k"]), W.to_f64(x["v"]),
                                                  x["scale"], rows)
    out, lse = ra.ring_sweep(qf, k, v, chunk_offsets=offs, scale=x["scale"])
    torch.cuda.synchronize()
    assert_close(out[:, rows], lse[:, :, rows], ref_out, ref_lse, f"sweep {name} ({len(rows)} rows)")
    if w.ring_anything:
        kp, pad = padded(x["k"], offs, 300.0)
        vp, _ = padded(x["v"], offs, -300.0)
        out2, lse2 = ra.ring_sweep(qf, dev(kp), dev(vp), chunk_offsets=offs, kv_chunk_stride=pad, scale=x["scale"])
        torch.cuda.synchronize()
        assert torch.equal(out, out2) and torch.equal(lse, lse2), "padded buffer changed the result"
