"""Engine cycles per 64-key tile of the 8-wave kernel's sweep, and the engine
clock while it runs, from the cycle-counter build of the library.

    python -m context_attention_diffusion_ringattn_amd.build --cycles
    python context_attention_diffusion_ringattn_amd/probes/sweep_cycles.py

The build compiles the same kernels with RINGATTN_CYCLE_COUNTERS: each
workgroup's first wave reads s_memtime (engine cycles) and s_memrealtime
(100 MHz reference ticks) after the prologue's barrier and before the
epilogue, and logs both with its tile count.  Here: the video-sized shard
at D = 128 (B=1, 8192 query rows, 65536 keys, 24 heads) and at D = 64 (48
heads, the same flops), one ringattn_forward per launch with 256 query rows
per workgroup and no K/V split, after a few seconds of warm-up launches so
that the clock has settled under the load.
"""

from __future__ import annotations

import ctypes
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
CYCLES_LIB = os.path.join(ROOT, "_build", "cycles", "libringattn.so")
os.environ["RINGATTN_LIB"] = CYCLES_LIB  # before the binding loads a library
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import context_attention_diffusion_ringattn_amd as ra  # noqa: E402
from context_attention_diffusion_ringattn_amd import _lib  # noqa: E402


def measure(heads: int, head_dim: int, warm_s: float = 3.0, seed: int = 0) -> dict:
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    sq, skv = 8192, 65536
    q = torch.randn((1, sq, heads, head_dim), device=dev, generator=g).to(torch.bfloat16)
    k = torch.randn((1, skv, heads, head_dim), device=dev, generator=g).to(torch.bfloat16)
    v = torch.randn((1, skv, heads, head_dim), device=dev, generator=g).to(torch.bfloat16)
    offs = [c * (skv // 8) for c in range(9)]
    scale = float(np.float32(1.0 / np.sqrt(head_dim)))

    def call():
        return ra.forward(q, k, v, chunk_offsets=offs, scale=scale, n_splits=1, block_m=256)

    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    call()
    e1.record()
    torch.cuda.synchronize()
    n_warm = max(3, int(warm_s * 1e3 / max(e0.elapsed_time(e1), 1e-3)))
    for _ in range(n_warm):
        call()
    e0.record()
    call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)

    lib = _lib.lib()
    lib.ringattn_cycle_log_slots.restype = ctypes.c_int
    lib.ringattn_cycle_log_read.restype = ctypes.c_int
    lib.ringattn_cycle_log_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    slots = lib.ringattn_cycle_log_slots()
    buf = np.zeros(slots * 4, dtype=np.uint64)
    if lib.ringattn_cycle_log_read(buf.ctypes.data, buf.nbytes) != 0:
        raise RuntimeError("reading the cycle log failed")
    rec = buf.reshape(slots, 4).astype(np.float64)
    grid = 8192 // 256 * heads
    rec = rec[:grid]
    cyc, ref, tiles = rec[:, 0], rec[:, 1], rec[:, 2]
    per_tile = cyc / tiles
    flops = 4.0 * sq * skv * head_dim * heads
    return {
        "heads": heads, "head_dim": head_dim, "workgroups": grid, "tiles_per_workgroup": float(tiles.mean()),
        "cycles_per_tile_mean": float(per_tile.mean()), "cycles_per_tile_min": float(per_tile.min()),
        "cycles_per_tile_max": float(per_tile.max()), "engine_clock_ghz": float((cyc / ref).mean() * 0.1),
        "launch_ms": ms, "tflops": flops / ms / 1e9,
    }


def main() -> int:
    if not torch.cuda.is_available():
        print("no ROCm device", file=sys.stderr)
        return 1
    if not os.path.exists(CYCLES_LIB):
        print(f"{CYCLES_LIB} is not built; run `python -m context_attention_diffusion_ringattn_amd.build --cycles`",
              file=sys.stderr)
        return 1
    print("| shard | workgroups x tiles | cycles per 64-key tile (mean, min-max) | engine clock | launch | TFLOP/s |")
    print("|---|---|---|---|---|---|")
    for heads, d in ((24, 128), (48, 64)):
        r = measure(heads, d)
        print(f"| video-sized, H={heads}, D={d} | {r['workgroups']} x {r['tiles_per_workgroup']:.0f} | "
              f"{r['cycles_per_tile_mean']:.0f} ({r['cycles_per_tile_min']:.0f}-{r['cycles_per_tile_max']:.0f}) | "
              f"{r['engine_clock_ghz']:.3f} GHz | {r['launch_ms']:.3f} ms | {r['tflops']:.1f} |", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
