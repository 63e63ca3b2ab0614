"""GPU parity: the HIP path against the fp64 oracle on the same bf16 inputs.

Tolerances (written here, used everywhere below): max |out - oracle| <= 1e-2
and max |lse - oracle| <= 1e-3, elementwise over every compared value.  Small
workloads are compared in full; the full-size Ulysses and video shards are run
in the launch configuration the benchmark times and compared on sampled rows
(every head) that the oracle computes one by one.
"""

import functools
import itertools
import math

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
    ra_mod._lib.lib()  # fail loudly if the library is missing
    return ra_mod


def dev(t):
    return t.to("cuda:0")


def errors(gpu_out, gpu_lse, ref_out, ref_lse):
    o = gpu_out.detach().to("cpu", torch.float64).numpy()
    l = gpu_lse.detach().to("cpu", torch.float64).numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), "non-finite GPU result"
    return float(np.max(np.abs(o - ref_out))), float(np.max(np.abs(l - ref_lse)))


def assert_close(gpu_out, gpu_lse, ref_out, ref_lse, what):
    eo, el = errors(gpu_out, gpu_lse, ref_out, ref_lse)
    print(f"{what}: max|dout|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= OUT_TOL, f"{what}: out error {eo}"
    assert el <= LSE_TOL, f"{what}: lse error {el}"


@functools.lru_cache(maxsize=None)
def workload_inputs(name):
    return W.make_inputs(name)


@functools.lru_cache(maxsize=None)
def workload_oracle(name):
    x = workload_inputs(name)
    return oracle.attention_fp64(W.to_f64(x["q"]), W.to_f64(x["k"]), W.to_f64(x["v"]), x["scale"])


@pytest.mark.parametrize("name", ["tiny", "flux", "ring_anything"])
def test_forward_small_workloads(ra, name):
    """Tiny, Flux-like and Ring Anything shards, compared in full, with the
    library's own partition and launch plan."""
    x = workload_inputs(name)
    w = x["workload"]
    print(f"case {name}: q{tuple(x['q'].shape)} kv{tuple(x['k'].shape)}", flush=True)
    offs = ra.chunk_offsets(w.seq_len, w.n_chunks, w.ring_anything)
    assert offs == oracle.chunk_offsets(w.seq_len, w.n_chunks, w.ring_anything)
    assert offs[1] == w.q_rows
    out, lse = ra.forward(dev(x["q"]), dev(x["k"]), dev(x["v"]), chunk_offsets=offs, scale=x["scale"])
    torch.cuda.synchronize()
    ref_out, ref_lse = workload_oracle(name)
    assert_close(out, lse, ref_out, ref_lse, f"forward {name}")


@pytest.mark.parametrize("name", ["flux", "ring_anything"])
@pytest.mark.parametrize("splits", [1, 2, 3, 7])
@pytest.mark.parametrize("block_m", [128, 256])
def test_forward_forced_splits(ra, name, splits, block_m):
    """Every split count and both workgroup shapes give the oracle's result
    (the last split of each query tile merges the partials by their LSE)."""
    x = workload_inputs(name)
    w = x["workload"]
    print(f"case {name} splits={splits} block_m={block_m}", flush=True)
    out, lse = ra.forward(dev(x["q"]), dev(x["k"]), dev(x["v"]), ring_degree=w.n_chunks,
                          ring_anything=w.ring_anything, scale=x["scale"], n_splits=splits, block_m=block_m)
    torch.cuda.synchronize()
    ref_out, ref_lse = workload_oracle(name)
    assert_close(out, lse, ref_out, ref_lse, f"forward {name} splits={splits} block_m={block_m}")


@pytest.mark.parametrize("name", ["tiny", "flux", "ring_anything"])
def test_step_path_matches_oracle_and_forward(ra, name):
    """The ring's own loop: accumulators initialised to (0, -inf), then one
    ringattn_step per chunk with the merge fused in the epilogue."""
    x = workload_inputs(name)
    w = x["workload"]
    print(f"case step {name}", flush=True)
    offs = oracle.chunk_offsets(w.seq_len, w.n_chunks, w.ring_anything)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    out_acc, lse_acc = ra.new_accumulators(q)
    for c in range(w.n_chunks):
        ra.step(q, k[:, offs[c]:offs[c + 1]].contiguous(), v[:, offs[c]:offs[c + 1]].contiguous(),
                out_acc, lse_acc, scale=x["scale"])
    torch.cuda.synchronize()
    ref_out, ref_lse = workload_oracle(name)
    assert_close(out_acc, lse_acc, ref_out, ref_lse, f"step path {name}")
    f_out, f_lse = ra.forward(q, k, v, chunk_offsets=offs, scale=x["scale"])
    torch.cuda.synchronize()
    assert_close(out_acc, lse_acc, f_out.cpu().double().numpy(), f_lse.cpu().double().numpy(),
                 f"step vs forward {name}")


def test_merge_api_and_empty_identity(ra):
    """ringattn_merge of two forward partials (disjoint key halves) equals the
    forward over all keys; a partial with lse = -inf and NaN output is the
    identity; two empties stay (0, -inf)."""
    x = workload_inputs("flux")
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    sc = x["scale"]
    a_out, a_lse = ra.forward(q, k[:, :2304].contiguous(), v[:, :2304].contiguous(), scale=sc)
    b_out, b_lse = ra.forward(q, k[:, 2304:].contiguous(), v[:, 2304:].contiguous(), scale=sc)
    ra.merge(a_out, a_lse, b_out, b_lse)
    torch.cuda.synchronize()
    ref_out, ref_lse = workload_oracle("flux")
    assert_close(a_out, a_lse, ref_out, ref_lse, "merge api")
    keep_out, keep_lse = a_out.clone(), a_lse.clone()
    junk_out = torch.full_like(a_out, float("nan"))
    junk_lse = torch.full_like(a_lse, float("-inf"))
    ra.merge(a_out, a_lse, junk_out, junk_lse)
    torch.cuda.synchronize()
    assert torch.equal(a_out, keep_out) and torch.equal(a_lse, keep_lse)
    e_out, e_lse = ra.new_accumulators(q)
    ra.merge(e_out, e_lse, junk_out.clone(), junk_lse.clone())
    torch.cuda.synchronize()
    assert torch.all(e_out == 0) and torch.all(e_lse == float("-inf"))
    ra.merge(e_out, e_lse, keep_out, keep_lse)
    torch.cuda.synchronize()
    assert torch.equal(e_out, keep_out) and torch.equal(e_lse, keep_lse)


def test_ring_anything_padded_buffer(ra):
    """Ring Anything's padded all-gather buffer (every chunk padded to 577 rows,
    padding filled with large garbage) gives the same result as the packed
    chunks: padding rows are excluded, never read as zeros."""
    x = workload_inputs("ring_anything")
    w = x["workload"]
    offs = oracle.chunk_offsets(w.seq_len, w.n_chunks, True)
    pad = oracle.padded_chunk_length(w.seq_len, w.n_chunks)
    B, S, H, D = x["k"].shape
    kp = torch.full((B, w.n_chunks * pad, H, D), 300.0, dtype=torch.bfloat16)
    vp = torch.full((B, w.n_chunks * pad, H, D), -300.0, dtype=torch.bfloat16)
    for c in range(w.n_chunks):
        n = offs[c + 1] - offs[c]
        kp[:, c * pad:c * pad + n] = x["k"][:, offs[c]:offs[c + 1]]
        vp[:, c * pad:c * pad + n] = x["v"][:, offs[c]:offs[c + 1]]
    ref_out, ref_lse = workload_oracle("ring_anything")
    for block_m in (128, 256):
        for splits in (0, 3):
            out, lse = ra.forward(dev(x["q"]), dev(kp), dev(vp), chunk_offsets=offs, kv_chunk_stride=pad,
                                  scale=x["scale"], n_splits=splits, block_m=block_m)
            torch.cuda.synchronize()
            assert_close(out, lse, ref_out, ref_lse, f"padded ring anything block_m={block_m} splits={splits}")


RAGGED_CASES = [
    # (B, H, D, Sq, chunk lengths, seed)
    (1, 1, 64, 1, [1], 100),
    (2, 3, 64, 77, [0, 33, 129, 1, 64, 65], 101),
    (1, 2, 128, 129, [200, 0, 0, 7], 102),
    (2, 1, 128, 300, [63, 64, 65, 127, 128, 129], 103),
    (1, 4, 128, 256, [1000], 104),
    (3, 2, 64, 45, [17] * 16, 105),
]


@pytest.mark.parametrize("case", RAGGED_CASES, ids=lambda c: f"B{c[0]}H{c[1]}D{c[2]}Sq{c[3]}n{len(c[4])}")
def test_ragged_shapes(ra, case):
    """Ragged query tails, ragged and empty chunks, both head dims, several
    batches, vs the oracle; also through the step path."""
    B, H, D, Sq, lens, seed = case
    S = sum(lens)
    x = W.make_random(B, Sq, S, H, D, seed, k_outlier_frac=0.05, k_outlier_scale=5.0)
    offs = [0]
    for n in lens:
        offs.append(offs[-1] + n)
    print(f"case ragged {case}", flush=True)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    ref_out, ref_lse = oracle.attention_fp64(W.to_f64(x["q"]), W.to_f64(x["k"]), W.to_f64(x["v"]), x["scale"])
    for block_m in (128, 256):
        for splits in (0, 1, 5):
            out, lse = ra.forward(q, k, v, chunk_offsets=offs, scale=x["scale"], n_splits=splits, block_m=block_m)
            torch.cuda.synchronize()
            assert_close(out, lse, ref_out, ref_lse, f"ragged forward block_m={block_m} splits={splits}")
        # the same chunks as a padded buffer (chunk table walked in the kernel)
        pad = max(max(lens), 1)
        kp = torch.full((B, len(lens) * pad, H, D), float("nan"), dtype=torch.bfloat16)
        vp = torch.full((B, len(lens) * pad, H, D), float("nan"), dtype=torch.bfloat16)
        for c in range(len(lens)):
            kp[:, c * pad:c * pad + lens[c]] = x["k"][:, offs[c]:offs[c + 1]]
            vp[:, c * pad:c * pad + lens[c]] = x["v"][:, offs[c]:offs[c + 1]]
        out, lse = ra.forward(q, dev(kp), dev(vp), chunk_offsets=offs, kv_chunk_stride=pad, scale=x["scale"],
                              block_m=block_m)
        torch.cuda.synchronize()
        assert_close(out, lse, ref_out, ref_lse, f"ragged padded block_m={block_m}")
    # the step path: the library's plan, then one split of 128 and of 256 rows
    # (the 8-wave kernel's in-place merge, staged through LDS at D = 128)
    for block_m in (0, 128, 256):
        out_acc, lse_acc = ra.new_accumulators(q)
        for c in range(len(lens)):
            ra.step(q, k[:, offs[c]:offs[c + 1]].contiguous(), v[:, offs[c]:offs[c + 1]].contiguous(),
                    out_acc, lse_acc, scale=x["scale"], n_splits=1, block_m=block_m)
        torch.cuda.synchronize()
        assert_close(out_acc, lse_acc, ref_out, ref_lse, f"ragged step path block_m={block_m}")


def test_no_keys_gives_empty_result(ra):
    x = W.make_random(1, 40, 0, 2, 64, 7)
    q = dev(x["q"])
    k = torch.empty((1, 0, 2, 64), dtype=torch.bfloat16, device="cuda:0")
    out, lse = ra.forward(q, k, k.clone(), chunk_offsets=[0, 0, 0], scale=x["scale"])
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(lse == float("-inf"))


def test_chunk_order_invariance(ra):
    """Reordering the chunks (a rank-rotated ring order) changes the result only
    by rounding."""
    x = workload_inputs("ring_anything")
    w = x["workload"]
    offs = oracle.chunk_offsets(w.seq_len, w.n_chunks, True)
    order = [3, 4, 5, 6, 7, 0, 1, 2]
    k = torch.cat([x["k"][:, offs[c]:offs[c + 1]] for c in order], dim=1)
    v = torch.cat([x["v"][:, offs[c]:offs[c + 1]] for c in order], dim=1)
    new_offs = [0]
    for c in order:
        new_offs.append(new_offs[-1] + offs[c + 1] - offs[c])
    out, lse = ra.forward(dev(x["q"]), dev(k), dev(v), chunk_offsets=new_offs, scale=x["scale"])
    torch.cuda.synchronize()
    ref_out, ref_lse = workload_oracle("ring_anything")
    assert_close(out, lse, ref_out, ref_lse, "rotated chunk order")


def test_deterministic(ra):
    """No atomics: repeated runs are bitwise identical (single split and split)."""
    x = workload_inputs("ring_anything")
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    for block_m in (128, 256):
        for splits in (1, 4):
            a = ra.forward(q, k, v, ring_degree=8, ring_anything=True, scale=x["scale"], n_splits=splits,
                           block_m=block_m)
            b = ra.forward(q, k, v, ring_degree=8, ring_anything=True, scale=x["scale"], n_splits=splits,
                           block_m=block_m)
            torch.cuda.synchronize()
            assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def sampled_rows(n_rows, count, extra=(), seed=0):
    rng = np.random.default_rng(seed)
    rows = set(int(r) for r in rng.choice(n_rows, size=min(count, n_rows), replace=False))
    rows.update([0, n_rows - 1])
    rows.update(int(r) for r in extra if 0 <= r < n_rows)
    return sorted(rows)


@pytest.mark.parametrize("name", ["ulysses", "video"])
def test_full_size_sampled(ra, name):
    """The full-size Ulysses share and video shard, run exactly as the benchmark
    runs them (library partition, automatic plan), compared on sampled query
    rows (all heads) including the outlier rows of the local shard."""
    x = W.make_inputs(name)
    w = x["workload"]
    print(f"case full-size {name}: q{tuple(x['q'].shape)} kv{tuple(x['k'].shape)}", flush=True)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    out, lse = ra.forward(q, k, v, ring_degree=w.n_chunks, ring_anything=w.ring_anything, scale=x["scale"])
    torch.cuda.synchronize()
    rows = sampled_rows(w.q_rows, 24, extra=x["q_outlier_rows"][:8], seed=w.seed)
    ref_out, ref_lse = oracle.attention_rows_fp64(W.to_f64(x["q"]), W.to_f64(x["k"]), W.to_f64(x["v"]),
                                                  x["scale"], rows)
    assert_close(out[:, rows], lse[:, :, rows], ref_out, ref_lse, f"{name} sampled rows {len(rows)}")


def test_invalid_call_writes_nothing(ra):
    """Every argument error the library reports (bad chunk offsets, a bad
    scale, a short workspace) is found before any launch: the output and
    accumulator buffers keep their contents."""
    x = workload_inputs("tiny")
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    out = torch.full((1, 128, 2, 64), 7.0, dtype=torch.float32, device="cuda:0")
    lse = torch.full((1, 2, 128), 7.0, dtype=torch.float32, device="cuda:0")
    qf = dev(x["q_full"])
    out_f = torch.full((1, 256, 2, 64), 7.0, dtype=torch.float32, device="cuda:0")
    lse_f = torch.full((1, 2, 256), 7.0, dtype=torch.float32, device="cuda:0")
    print("case invalid calls", flush=True)
    for bad in ([0, 200, 100, 256], [1, 128, 256], [0, -1, 256]):
        with pytest.raises(ra.RingAttnError):
            ra.forward(q, k, v, chunk_offsets=bad, scale=x["scale"], out=out, lse=lse)
        with pytest.raises(ra.RingAttnError):
            ra.ring_sweep(qf, k, v, chunk_offsets=bad, scale=x["scale"], out=out_f, lse=lse_f)
    for bad_scale in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(ra.RingAttnError):
            ra.forward(q, k, v, chunk_offsets=[0, 128, 256], scale=bad_scale, out=out, lse=lse)
    short = torch.empty((16,), dtype=torch.uint8, device="cuda:0")
    with pytest.raises(ra.RingAttnError):
        ra.forward(q, k, v, chunk_offsets=[0, 128, 256], scale=x["scale"], n_splits=2, out=out, lse=lse,
                   workspace=short)
    acc_o, acc_l = out.clone(), lse.clone()
    with pytest.raises(ra.RingAttnError):
        ra.step(q, k[:, :128].contiguous(), v[:, :128].contiguous(), acc_o, acc_l, scale=float("nan"))
    torch.cuda.synchronize()
    for t in (out, lse, out_f, lse_f, acc_o, acc_l):
        assert torch.all(t == 7.0)


@pytest.mark.parametrize("name", ["ring_even", "ulysses_even"])
def test_even_counterparts(ra, name):
    """The plain-split counterparts of the Ring Anything and Ulysses Anything
    workloads, compared in full (ring) or on sampled rows (Ulysses)."""
    x = workload_inputs(name)
    w = x["workload"]
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    out, lse = ra.forward(q, k, v, ring_degree=w.n_chunks, scale=x["scale"])
    torch.cuda.synchronize()
    rows = list(range(w.q_rows)) if name == "ring_even" else sampled_rows(w.q_rows, 24, seed=w.seed)
    ref_out, ref_lse = oracle.attention_rows_fp64(W.to_f64(x["q"]), W.to_f64(x["k"]), W.to_f64(x["v"]),
                                                  x["scale"], rows)
    assert_close(out[:, rows], lse[:, :, rows], ref_out, ref_lse, name)


def test_maximum_chunk_count_and_wide_heads(ra):
    """The largest chunk table the ABI accepts (RINGATTN_MAX_CHUNKS chunks of
    mixed lengths, some empty) through the packed and the padded layout, and
    a layer with many heads; both workgroup shapes."""
    n = ra._lib.RINGATTN_MAX_CHUNKS
    rng = np.random.default_rng(77)
    lens = [0 if rng.random() < 0.15 else int(rng.integers(1, 41)) for _ in range(n)]
    S = sum(lens)
    offs = [0]
    for m in lens:
        offs.append(offs[-1] + m)
    for B, H, D, Sq in ((1, 3, 128, 300), (2, 40, 64, 70)):
        print(f"case max chunks: B={B} H={H} D={D} Sq={Sq} S={S} n={n}", flush=True)
        x = W.make_random(B, Sq, S, H, D, 78 + H, k_outlier_frac=0.02, k_outlier_scale=6.0)
        ref_out, ref_lse = oracle.attention_fp64(W.to_f64(x["q"]), W.to_f64(x["k"]), W.to_f64(x["v"]), x["scale"])
        q = dev(x["q"])
        pad = max(lens)
        kp = torch.full((B, n * pad, H, D), float("nan"), dtype=torch.bfloat16)
        vp = torch.full((B, n * pad, H, D), float("nan"), dtype=torch.bfloat16)
        for c in range(n):
            kp[:, c * pad:c * pad + lens[c]] = x["k"][:, offs[c]:offs[c + 1]]
            vp[:, c * pad:c * pad + lens[c]] = x["v"][:, offs[c]:offs[c + 1]]
        for block_m in (128, 256):
            out, lse = ra.forward(q, dev(x["k"]), dev(x["v"]), chunk_offsets=offs, scale=x["scale"], block_m=block_m)
            torch.cuda.synchronize()
            assert_close(out, lse, ref_out, ref_lse, f"max chunks packed block_m={block_m} H={H}")
            out, lse = ra.forward(q, dev(kp), dev(vp), chunk_offsets=offs, kv_chunk_stride=pad, scale=x["scale"],
                                  block_m=block_m, n_splits=3)
            torch.cuda.synchronize()
            assert_close(out, lse, ref_out, ref_lse, f"max chunks padded block_m={block_m} H={H}")
