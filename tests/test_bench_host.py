"""Host-side logic of bench.py and the input generator, on the CPU: the
single-GPU guard, the counted-traffic lookup and its staleness check, and
the workload shapes, flop counts and seeding."""

import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from context_attention_diffusion_ringattn_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_record_is_used_only_while_fresh(tmp_path, monkeypatch):
    """The counted HBM bytes are reported only for the counted kernel and
    workload, and only while every source the record lists is unchanged."""
    import hashlib
    src = tmp_path / "k" / "kernel.hip"
    src.parent.mkdir(parents=True)
    src.write_text("// kernel source\n")
    (tmp_path / "profiles").mkdir()
    rec = {"kernel_sources": ["k/kernel.hip"],
           "kernel_sources_sha256": hashlib.sha256(src.read_bytes()).hexdigest(),
           "hbm_bytes_per_launch": 1234567.6}
    (tmp_path / "profiles" / "attn_pp_video_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_from_profiles("video", 256) == 1234568
    assert bench.traffic_from_profiles("video", 128) is None      # another kernel
    assert bench.traffic_from_profiles("flux", 256) is None       # no record for this workload
    src.write_text("// kernel source, edited\n")
    assert bench.traffic_from_profiles("video", 256) is None      # stale


def test_committed_record_names_existing_sources():
    with open(os.path.join(ROOT, "profiles", "attn_pp_video_traffic.json")) as f:
        rec = json.load(f)
    assert all(os.path.exists(os.path.join(ROOT, p)) for p in rec["kernel_sources"])
    assert rec["hbm_bytes_per_launch"] > 957e6   # at least the algorithmic bytes


@pytest.mark.parametrize("name,q_shape,kv_shape,flops", [
    ("tiny", (1, 128, 2, 64), (1, 256, 2, 64), 4 * 128 * 256 * 64 * 2),
    ("flux", (1, 1152, 24, 128), (1, 4608, 24, 128), 4 * 1152 * 4608 * 128 * 24),
    ("ring_anything", (1, 577, 24, 128), (1, 4611, 24, 128), 4 * 577 * 4611 * 128 * 24),
    ("ulysses", (1, 16384, 6, 128), (1, 16384, 6, 128), 4 * 16384 * 16384 * 128 * 6),
    ("ulysses_anything", (1, 4481, 6, 128), (1, 4481, 6, 128), 4 * 4481 * 4481 * 128 * 6),
])
def test_workload_shapes_and_flops(name, q_shape, kv_shape, flops):
    x = W.make_inputs(name)
    w = x["workload"]
    assert tuple(x["q"].shape) == q_shape and tuple(x["k"].shape) == kv_shape == tuple(x["v"].shape)
    assert x["q"].dtype == x["k"].dtype == torch.bfloat16
    assert w.flops == flops
    assert x["scale"] == float(np.float32(1.0 / np.sqrt(q_shape[-1])))


def test_large_workload_definitions():
    for name, q_rows, seq, heads, chunks in [("video", 8192, 65536, 24, 8), ("usp", 16384, 65536, 12, 4)]:
        w = W.WORKLOADS[name]
        assert (w.q_rows, w.seq_len, w.heads, w.n_chunks, w.head_dim) == (q_rows, seq, heads, chunks, 128)
        assert w.flops == 4 * q_rows * seq * 128 * heads


def test_inputs_are_seeded_and_local_shard_is_rank0():
    a, b = W.make_inputs("ring_anything"), W.make_inputs("ring_anything")
    assert torch.equal(a["q_full"], b["q_full"]) and torch.equal(a["k"], b["k"]) and torch.equal(a["v"], b["v"])
    assert torch.equal(a["q"], a["q_full"][:, :577])
    # 1 % of the 4611 K rows were scaled by 8 before rounding
    assert len(a["k_outlier_rows"]) == round(0.01 * 4611)
    norms = a["k_f32"][0].reshape(4611, -1).std(axis=1)
    assert np.all(norms[a["k_outlier_rows"]] > 4.0)
    c = W.make_inputs("flux")
    assert not torch.equal(c["k"][:, :577], a["k"][:, :577])


def test_cpu_baseline_pool_matches_oracle():
    """The oracle timed over the worker pool gives the same rows as one call
    of the oracle, and reports the worker count as its cores."""
    import oracle
    x = W.make_inputs("tiny")
    pool, n = bench.make_oracle_pool(x)
    try:
        cb, rows, out, lse = bench.cpu_baseline(x, 0.2, pool, n)
    finally:
        pool.close()
        pool.join()
    assert cb["kind"] == "oracle" and cb["cores"] == n == bench.oracle_workers() and cb["value"] > 0
    ref_out, ref_lse = oracle.attention_rows_fp64(W.to_f64(x["q"]), W.to_f64(x["k"]), W.to_f64(x["v"]),
                                                  x["scale"], rows)
    assert np.array_equal(out, ref_out) and np.array_equal(lse, ref_lse)
