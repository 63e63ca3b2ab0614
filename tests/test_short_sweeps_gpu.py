"""The 256-row kernel on short sweeps: 1-5 tiles of 64 keys, full and
ragged, at D = 64 and 128, through every epilogue it has.

Its MFMA phase is one software pipeline: step 0 (the QK of the first tile)
runs on its own, and the last step (the PV of the last tile) still reads the
first K operands of a QK that does not run.  These cases keep the sweep
short enough that those two steps are most of it: a one-tile sweep is
nothing but them, and a split plan over one or two tiles leaves some splits
with no tile at all.  Each result is compared with the fp64 oracle on the
same bf16 inputs, to the tolerances of the other parity tests:
max|dout| <= 1e-2, max|dlse| <= 1e-3."""

import numpy as np
import pytest
import torch

import oracle
from context_attention_diffusion_ringattn_amd import workloads as W

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2
LSE_TOL = 1e-3

# key counts: 1, 2, 3 and 5 tiles of 64 keys, full and with a ragged tail
KEY_COUNTS = [1, 64, 65, 128, 150, 192, 300]


@pytest.fixture(scope="module")
def ra():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    import context_attention_diffusion_ringattn_amd as ra_mod
    ra_mod._lib.lib()
    return ra_mod


def check(out, lse, ref_out, ref_lse, what):
    o = out.detach().to("cpu", torch.float64).numpy()
    l = lse.detach().to("cpu", torch.float64).numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), f"{what}: non-finite result"
    eo, el = float(np.max(np.abs(o - ref_out))), float(np.max(np.abs(l - ref_lse)))
    print(f"{what}: max|dout|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= OUT_TOL and el <= LSE_TOL, f"{what}: out {eo}, lse {el}"


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("n_keys", KEY_COUNTS)
def test_short_sweeps(ra, D, n_keys):
    B, H, Sq = 1, 2, 300  # two query tiles of 256 rows, the second ragged
    x = W.make_random(B, Sq, n_keys, H, D, 4000 + 7 * n_keys + D, k_outlier_frac=0.05, k_outlier_scale=5.0)
    ref_out, ref_lse = oracle.attention_fp64(W.to_f64(x["q"]), W.to_f64(x["k"]), W.to_f64(x["v"]), x["scale"])
    q, k, v = (x[n].to("cuda:0") for n in ("q", "k", "v"))
    offs = [0, n_keys]
    tag = f"D={D} keys={n_keys}"
    print(f"case {tag}", flush=True)

    # Final epilogue (one split) and Partial epilogues + merge (two and three splits)
    for splits in (1, 2, 3):
        out, lse = ra.forward(q, k, v, chunk_offsets=offs, scale=x["scale"], n_splits=splits, block_m=256)
        torch.cuda.synchronize()
        check(out, lse, ref_out, ref_lse, f"forward {tag} splits={splits}")

    # the chunk-table walk: the keys as two chunks of a NaN-padded buffer
    c0 = n_keys // 2
    lens = [c0, n_keys - c0]
    pad = max(lens)
    kp = torch.full((B, 2 * pad, H, D), float("nan"), dtype=torch.bfloat16)
    vp = torch.full_like(kp, float("nan"))
    kp[:, :lens[0]] = x["k"][:, :c0]
    vp[:, :lens[0]] = x["v"][:, :c0]
    kp[:, pad:pad + lens[1]] = x["k"][:, c0:]
    vp[:, pad:pad + lens[1]] = x["v"][:, c0:]
    out, lse = ra.forward(q, kp.to("cuda:0"), vp.to("cuda:0"), chunk_offsets=[0, c0, n_keys], kv_chunk_stride=pad,
                          scale=x["scale"], n_splits=1, block_m=256)
    torch.cuda.synchronize()
    check(out, lse, ref_out, ref_lse, f"padded {tag}")

    # Accum epilogue: the ring step into an accumulator that already holds
    # the first chunk's partial (so the in-place merge weighs both sides)
    out_acc, lse_acc = ra.new_accumulators(q)
    for lo, hi in ((0, c0), (c0, n_keys)):
        ra.step(q, k[:, lo:hi].contiguous(), v[:, lo:hi].contiguous(), out_acc, lse_acc, scale=x["scale"],
                n_splits=1, block_m=256)
    torch.cuda.synchronize()
    check(out_acc, lse_acc, ref_out, ref_lse, f"step {tag}")
