#!/usr/bin/env python3
"""Benchmark one GPU's share of ring attention on an MI355X.

A step is one full pass of the shard: the local Q rows attend to every K/V
chunk and the float32 output + LSE are produced (``ringattn_forward``: all
chunk passes, the LSE merge and, if planned, the split merge).  With
``--sweep`` a step is the whole ring on this GPU (``ringattn_ring_sweep``):
every rank's rows, each rank visiting the chunks in its rotated order with a
float32 merge per step.  Inputs are seeded synthetic bf16 tensors already
resident in HBM when timing starts.

Prints ONE JSON line.  ``value`` is attention TFLOP/s = 4*B*Sq*Skv*D*H /
seconds per step.  ``roofline`` reports the attention kernel against the
published MI355X dense bf16 MFMA peak (2.5 PFLOP/s), with its duration taken
from HIP events on the stream the kernel is launched on.  ``cpu_baseline``
times the fp64 oracle on a bounded sample of query rows on the host cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s (4·Sq·Skv·D·H) per ring shard on 1 MI355X; % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X published dense bf16 MFMA peak
PEAK_HBM_GBS = 8000.0


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200,
                    help="timed steps (default 200: about 1.1 s of kernels on the video shard)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="video",
                    help="tiny | flux | ring_anything | ring_even | ulysses | ulysses_anything | ulysses_even | usp | video (default: video)")
    ap.add_argument("--splits", type=int, default=0, help="force the K/V split count (0 = library plan)")
    ap.add_argument("--block-m", type=int, default=0, help="force query rows per workgroup, 128 or 256 "
                                                            "(0 = library plan)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate host time spent timing the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="time the whole ring on this GPU instead of one shard: every rank's query rows, each "
                         "rank visiting the chunks in its rotated order with a float32 merge per step")
    ap.add_argument("--ring-steps", action="store_true",
                    help="time the ring's own loop on this shard instead of one forward call: accumulator "
                         "initialisation plus one split ring step (ringattn_step_split, library plan) per chunk")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step (all of its launches) in a HIP graph once and time its replays")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (calibrates the HBM byte "
                         "counters of a profiler run) and exit")
    return ap.parse_args()


def copy_probe(mib: int) -> None:
    """A plain copy kernel of known size: reads and writes mib MiB once."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "launches": 3}),
          flush=True)


def traffic_from_profiles(workload: str, block_m: int):
    """HBM bytes per launch of the attention kernel, from the committed
    rocprofv3 counter record profiles/attn_pp_<workload>_traffic.json
    (FETCH_SIZE and WRITE_SIZE scaled by a plain copy of known size).

    None when there is no record for this workload, when the plan launches a
    different kernel than the one counted, or when any source the record
    lists has changed since the counters were taken (its sha256 differs)."""
    if block_m != 256:
        return None
    path = os.path.join(ROOT, "profiles", f"attn_pp_{workload}_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        h = hashlib.sha256()
        for src in rec["kernel_sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != rec["kernel_sources_sha256"]:
            return None
        return int(round(rec["hbm_bytes_per_launch"]))
    except (OSError, ValueError, KeyError):
        return None


# Inputs the oracle workers read: set in the parent before the pool forks, so
# every worker inherits them copy-on-write instead of receiving them pickled.
_ORACLE_INPUTS = {}


def _oracle_worker_init():
    """One BLAS thread per worker process: the pool supplies the parallelism."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # threadpoolctl missing: BLAS keeps its own count
        pass


def _oracle_task(task):
    """The oracle on query rows `rows` of head h (all keys), in its own process."""
    import numpy as np

    import oracle

    h, rows = task
    x = _ORACLE_INPUTS
    q = x["q"][:, rows, h:h + 1, :].astype(np.float64)
    k = x["k"][:, :, h:h + 1, :].astype(np.float64)
    v = x["v"][:, :, h:h + 1, :].astype(np.float64)
    out, lse = oracle.attention_fp64(q, k, v, x["scale"])
    return h, rows, out, lse


def oracle_workers() -> int:
    """Worker processes for the oracle: the host cores this process may run
    on, at most 16 (the host's CPU share per GPU)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def make_oracle_pool(x, q_key: str = "q"):
    """Fork the oracle's worker pool.  Called before the GPU is touched, so
    the workers are plain CPU processes holding the bf16 inputs as float32."""
    import multiprocessing as mp

    _ORACLE_INPUTS.clear()
    _ORACLE_INPUTS.update(q=x[q_key].float().numpy(), k=x["k"].float().numpy(), v=x["v"].float().numpy(),
                          scale=x["scale"])
    n = oracle_workers()
    return mp.get_context("fork").Pool(n, initializer=_oracle_worker_init), n


def cpu_baseline(x, target_s: float, pool, n_workers: int, q_key: str = "q"):
    """Time the oracle on a sample of query rows of x[q_key] (all heads, all
    keys), spread over the worker pool as (head, row block) tasks."""
    import numpy as np

    w = x["workload"]
    n_rows = x[q_key].shape[1]
    rng = np.random.default_rng(1234)

    def run(n):
        rows = sorted(int(r) for r in rng.choice(n_rows, size=min(n, n_rows), replace=False))
        blk = max(1, -(-len(rows) * w.heads // (4 * n_workers)))  # about four tasks per worker
        blk = min(blk, 256)
        tasks = [(h, rows[i:i + blk]) for h in range(w.heads) for i in range(0, len(rows), blk)]
        out = np.zeros((w.batch, len(rows), w.heads, w.head_dim))
        lse = np.zeros((w.batch, w.heads, len(rows)))
        pos = {r: i for i, r in enumerate(rows)}
        t0 = time.perf_counter()
        for h, rr, o, l in pool.imap_unordered(_oracle_task, tasks):
            idx = [pos[r] for r in rr]
            out[:, idx, h, :] = o[:, :, 0, :]
            lse[:, h, idx] = l[:, 0, :]
        return rows, out, lse, time.perf_counter() - t0

    run(min(n_workers, n_rows))                 # worker start-up, page faults
    n0 = min(4 * n_workers, n_rows)
    _, _, _, t0 = run(n0)
    while t0 < target_s / 8 and n0 < n_rows:    # calibrate on a sample long enough to time
        n0 = min(n_rows, 4 * n0)
        _, _, _, t0 = run(n0)
    n = int(max(n0, min(n_rows, n0 * target_s / max(t0, 1e-3))))
    rows, out, lse, t = run(n)
    flops = 4.0 * w.batch * len(rows) * w.seq_len * w.head_dim * w.heads
    return {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        "cores": int(n_workers),
        "kind": "oracle",
        "sample": f"{len(rows)} of {n_rows} query rows x {w.heads} heads x {w.seq_len} keys "
                  f"(fp64 NumPy, {t:.1f} s wall on {n_workers} worker processes with one BLAS thread each; "
                  f"{len(os.sched_getaffinity(0))} host cores in this process's affinity)",
    }, rows, out, lse


def main():
    args = parse_args()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's ring shard only; the library has no multi-GPU path "
              "(the K/V exchange between GPUs is not built). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import context_attention_diffusion_ringattn_amd as ra
    from context_attention_diffusion_ringattn_amd import workloads as W

    # device_count() does not initialise the GPU (is_available() does), so the
    # oracle's pool below is still forked from a process with no GPU state.
    if torch.cuda.device_count() < 1:
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    x = W.make_inputs(args.workload)
    w = x["workload"]
    q_key = "q_full" if args.sweep else "q"
    pool = None
    if not args.no_cpu_baseline:
        pool, n_workers = make_oracle_pool(x, q_key)   # forked before any GPU call
    dev = torch.device("cuda:0")
    q, k, v = x[q_key].to(dev), x["k"].to(dev), x["v"].to(dev)
    n_q = q.shape[1]
    offs = ra.chunk_offsets(w.seq_len, w.n_chunks, w.ring_anything)
    out = torch.empty((w.batch, n_q, w.heads, w.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((w.batch, w.heads, n_q), dtype=torch.float32, device=dev)
    if args.sweep:
        # each ring step of each rank is a single-split launch of the library's plan
        n_splits, block_m, ws_bytes = 1, ra.forward_plan((w.batch, offs[1], w.heads, w.head_dim),
                                                         [0, offs[1] - offs[0]], 1)[1], 0
        ws = None

        def step():
            ra.ring_sweep(q, k, v, chunk_offsets=offs, scale=x["scale"], out=out, lse=lse)
    elif args.ring_steps:
        # every chunk's step with the library's plan for its length; one workspace fits the largest
        plans = [ra.step_plan(tuple(q.shape), offs[c + 1] - offs[c], args.splits, args.block_m)
                 for c in range(w.n_chunks)]
        ws = ra.new_workspace(max(p[2] for p in plans), dev)
        n_splits, block_m = plans[0][0], plans[0][1]
        chunks = [(k[:, offs[c]:offs[c + 1]], v[:, offs[c]:offs[c + 1]]) for c in range(w.n_chunks)]
        assert all(kc.is_contiguous() for kc, _ in chunks), "chunk views must be contiguous (batch 1)"

        def step():
            ra.acc_init(out, lse)
            for (kc, vc), (sp, bm, _) in zip(chunks, plans):
                ra.step(q, kc, vc, out, lse, scale=x["scale"], n_splits=sp, block_m=bm, workspace=ws)
    else:
        n_splits, block_m, ws_bytes = ra.forward_plan(tuple(q.shape), offs, args.splits, args.block_m)
        ws = ra.new_workspace(ws_bytes, dev)

        def step():
            ra.forward(q, k, v, chunk_offsets=offs, scale=x["scale"], n_splits=n_splits, block_m=block_m,
                       out=out, lse=lse, workspace=ws)

    if args.graph:
        # The library enqueues kernels on torch's current stream and nothing
        # else, so a step captures as it is; one eager run on a side stream
        # first, as capture requires.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        step = graph.replay
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The library launches on torch's current stream; the events go on the same
    # stream.  The timed region holds the K steps back to back between one pair
    # of events (an event between steps costs a few microseconds of GPU time,
    # which is visible on the smaller shards).
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    avg_ms = ev0.elapsed_time(ev1) / args.steps
    # Spread of single steps, from a second pass with an event pair per step.
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    per_step_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    flops = 4.0 * w.batch * n_q * w.seq_len * w.head_dim * w.heads
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (avg_ms * 1e-3) / 1e12

    traffic = None if (args.sweep or args.ring_steps) else traffic_from_profiles(args.workload, block_m)
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"{w.name}_ring_sweep" if args.sweep else (f"{w.name}_ring_steps" if args.ring_steps
                                                                     else w.name)) + ("_graph" if args.graph else ""),
            "description": (f"every rank of the ring on one GPU ({w.n_chunks} ranks, rank-rotated chunk order, "
                            f"float32 merge per step); " if args.sweep else "")
                           + (f"the ring's loop: accumulator init + {w.n_chunks} split ring steps; "
                              if args.ring_steps else "")
                           + ("each step's launches replayed from one HIP graph; " if args.graph else "")
                           + w.description,
            "batch": w.batch, "heads": w.heads, "head_dim": w.head_dim,
            "q_rows": n_q, "kv_rows": w.seq_len, "n_chunks": w.n_chunks,
            "ring_anything": w.ring_anything,
            "flops_per_step": flops,
            "splits": n_splits,
            "block_m": block_m,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel_ms": {"mean": round(avg_ms, 4), "median": round(float(np.median(per_step_ms)), 4),
                          "min": round(float(np.min(per_step_ms)), 4)},
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        cb, rows, ref_out, ref_lse = cpu_baseline(x, args.cpu_seconds, pool, n_workers, q_key)
        pool.close()
        pool.join()
        result["cpu_baseline"] = cb
        o = out[:, rows].detach().cpu().double().numpy()
        l = lse[:, :, rows].detach().cpu().double().numpy()
        result["parity"] = {"rows_checked": len(rows),
                            "max_abs_err_out": float(np.max(np.abs(o - ref_out))),
                            "max_abs_err_lse": float(np.max(np.abs(l - ref_lse)))}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
