"""Seeded random parity cases on the GPU: shapes, chunk layouts, launch plans
and scales drawn from a fixed generator, each compared with the oracle's
one-shot fp64 attention (max |out - oracle| <= 1e-2, max |lse - oracle| <=
1e-3).

Each case draws batch 1-3, heads 1-6, head_dim 64 or 128, 1-400 query rows,
1-12 chunks of 0-300 keys (about one in five empty), the packed or the
padded (NaN-filled) K/V buffer, the query rows per workgroup (library
choice, 128 or 256), the K/V split count (library choice, 1, 2, 3 or 7) and
the scale (1/sqrt(head_dim) or a value in [0.02, 0.3]).  Every third case
also runs the ring's own loop (accumulator init + one step per chunk), and
every fourth the whole ring on one GPU when the query length equals the key
length.
"""

import numpy as np
import pytest
import torch

import oracle
from context_attention_diffusion_ringattn_amd import workloads as W

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2
LSE_TOL = 1e-3
N_CASES = 32


@pytest.fixture(scope="module")
def ra():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    import context_attention_diffusion_ringattn_amd as ra_mod
    ra_mod._lib.lib()
    return ra_mod


def draw_case(i):
    rng = np.random.Generator(np.random.PCG64(1000 + i))
    B = int(rng.integers(1, 4))
    H = int(rng.integers(1, 7))
    D = int(rng.choice([64, 128]))
    Sq = int(rng.integers(1, 401))
    n = int(rng.integers(1, 13))
    lens = [0 if rng.random() < 0.2 else int(rng.integers(1, 301)) for _ in range(n)]
    padded = bool(rng.random() < 0.4)
    block_m = int(rng.choice([0, 128, 256]))
    splits = int(rng.choice([0, 1, 2, 3, 7]))
    scale = None if rng.random() < 0.5 else float(np.float32(rng.uniform(0.02, 0.3)))
    return dict(B=B, H=H, D=D, Sq=Sq, lens=lens, padded=padded, block_m=block_m, splits=splits, scale=scale,
                seed=2000 + i)


def assert_close(o, l, ref_o, ref_l, what):
    o = o.detach().to("cpu", torch.float64).numpy()
    l = l.detach().to("cpu", torch.float64).numpy()
    finite = np.isfinite(ref_l)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    assert np.array_equal(np.isfinite(l), finite), f"{what}: -inf pattern of the LSE differs"
    eo = float(np.max(np.abs(o - ref_o))) if o.size else 0.0
    el = float(np.max(np.abs(l[finite] - ref_l[finite]))) if finite.any() else 0.0
    print(f"{what}: max|dout|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= OUT_TOL, f"{what}: out error {eo}"
    assert el <= LSE_TOL, f"{what}: lse error {el}"


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(ra, i):
    c = draw_case(i)
    B, H, D, Sq, lens = c["B"], c["H"], c["D"], c["Sq"], c["lens"]
    S = sum(lens)
    print(f"case random {i}: {c}", flush=True)
    x = W.make_random(B, Sq, S, H, D, c["seed"], k_outlier_frac=0.03, k_outlier_scale=6.0)
    scale = c["scale"] if c["scale"] is not None else x["scale"]
    offs = [0]
    for n in lens:
        offs.append(offs[-1] + n)
    ref_out, ref_lse = oracle.attention_fp64(W.to_f64(x["q"]), W.to_f64(x["k"]), W.to_f64(x["v"]), scale)
    q = x["q"].to("cuda:0")
    if c["padded"]:
        pad = max(max(lens), 1)
        kp = torch.full((B, len(lens) * pad, H, D), float("nan"), dtype=torch.bfloat16)
        vp = torch.full((B, len(lens) * pad, H, D), float("nan"), dtype=torch.bfloat16)
        for j in range(len(lens)):
            kp[:, j * pad:j * pad + lens[j]] = x["k"][:, offs[j]:offs[j + 1]]
            vp[:, j * pad:j * pad + lens[j]] = x["v"][:, offs[j]:offs[j + 1]]
        out, lse = ra.forward(q, kp.to("cuda:0"), vp.to("cuda:0"), chunk_offsets=offs, kv_chunk_stride=pad,
                              scale=scale, n_splits=c["splits"], block_m=c["block_m"])
    else:
        out, lse = ra.forward(q, x["k"].to("cuda:0"), x["v"].to("cuda:0"), chunk_offsets=offs, scale=scale,
                              n_splits=c["splits"], block_m=c["block_m"])
    torch.cuda.synchronize()
    assert_close(out, lse, ref_out, ref_lse, f"random {i} forward")
    if i % 3 == 0:
        k, v = x["k"].to("cuda:0"), x["v"].to("cuda:0")
        o_acc, l_acc = ra.new_accumulators(q)
        for j in range(len(lens)):
            ra.step(q, k[:, offs[j]:offs[j + 1]].contiguous(), v[:, offs[j]:offs[j + 1]].contiguous(), o_acc, l_acc,
                    scale=scale)
        torch.cuda.synchronize()
        assert_close(o_acc, l_acc, ref_out, ref_lse, f"random {i} step path")


@pytest.mark.parametrize("i", range(0, N_CASES, 4))
def test_random_sweep(ra, i):
    """The whole ring on one GPU for the case's chunk lengths (query rows =
    every key row), against one-shot attention over all keys."""
    c = draw_case(i)
    B, H, D, lens = c["B"], c["H"], c["D"], c["lens"]
    S = sum(lens)
    if S == 0:
        pytest.skip("no keys: the ring has no query rows")
    print(f"case random sweep {i}: {c}", flush=True)
    x = W.make_random(B, S, S, H, D, c["seed"] + 500, k_outlier_frac=0.03, k_outlier_scale=6.0)
    scale = c["scale"] if c["scale"] is not None else x["scale"]
    offs = [0]
    for n in lens:
        offs.append(offs[-1] + n)
    ref_out, ref_lse = oracle.attention_fp64(W.to_f64(x["q"]), W.to_f64(x["k"]), W.to_f64(x["v"]), scale)
    out, lse = ra.ring_sweep(x["q"].to("cuda:0"), x["k"].to("cuda:0"), x["v"].to("cuda:0"), chunk_offsets=offs,
                             scale=scale)
    torch.cuda.synchronize()
    assert_close(out, lse, ref_out, ref_lse, f"random {i} sweep")
