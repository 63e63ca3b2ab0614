"""The 128-row kernel's two-key-group form: a launch with at most one
workgroup per compute unit runs each workgroup as two groups of four waves
that sweep alternate 32-key tiles and merge their partial states through LDS
before the epilogue.  These cases pin that form to the fp64 oracle where the
groups' tile counts differ or the second group has no tile at all (1-5
tiles, ragged tails), on packed and NaN-padded K/V, at D = 64 and 128, for
the forward call (Final and split Partial epilogues) and the ring step
(Accum epilogue).  Tolerances as in test_parity_gpu: max|dout| <= 1e-2,
max|dlse| <= 1e-3 against the fp64 oracle on the same bf16 inputs."""

import numpy as np
import pytest
import torch

import oracle

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


def draw(seed, B, Sq, Skv, H, D):
    rng = np.random.default_rng(seed)
    f = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32)).to(torch.bfloat16)
    return f(B, Sq, H, D), f(B, Skv, H, D), f(B, Skv, H, D)


def f64(t):
    return t.to(torch.float64).numpy()


def check(out, lse, ref_out, ref_lse, what):
    o = out.detach().to("cpu", torch.float64).numpy()
    l = lse.detach().to("cpu", torch.float64).numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), f"{what}: non-finite result"
    eo, el = float(np.max(np.abs(o - ref_out))), float(np.max(np.abs(l - ref_lse)))
    print(f"{what}: max|dout|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= OUT_TOL and el <= LSE_TOL, f"{what}: out {eo}, lse {el}"


# (query rows, key lengths of the chunks): 128-row query tiles x 1-3 heads
# keep every launch at no more workgroups than compute units.
CASES = [
    (100, [17]),            # one ragged tile: the second group has none
    (128, [32]),            # one full tile
    (200, [33]),            # two tiles, the second ragged: one each
    (128, [96]),            # three tiles: 2 and 1
    (250, [130]),           # five tiles, ragged tail: 3 and 2
    (128, [40, 7, 64]),     # three chunks (5 tiles when chunk-aligned)
]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"Sq{c[0]}-" + "_".join(map(str, c[1])))
@pytest.mark.parametrize("padded", [False, True])
def test_key_groups_forward(ra, D, case, padded):
    Sq, lens = case
    B, H = 1, 3
    offs = [0]
    for n in lens:
        offs.append(offs[-1] + n)
    Skv = offs[-1]
    q, k, v = draw(1000 + Sq + Skv + D, B, Sq, Skv, H, D)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    ref_out, ref_lse = oracle.attention_fp64(f64(q), f64(k), f64(v), scale)
    if padded:
        pad = max(lens)
        kp = torch.full((B, len(lens) * pad, H, D), float("nan"), dtype=torch.bfloat16)
        vp = torch.full_like(kp, float("nan"))
        for c, n in enumerate(lens):
            kp[:, c * pad:c * pad + n] = k[:, offs[c]:offs[c + 1]]
            vp[:, c * pad:c * pad + n] = v[:, offs[c]:offs[c + 1]]
        kk, vv, stride = kp.cuda(), vp.cuda(), pad
    else:
        kk, vv, stride = k.cuda(), v.cuda(), 0
    for splits in (1, 2):
        print(f"case D={D} Sq={Sq} lens={lens} padded={padded} splits={splits}", flush=True)
        out, lse = ra.forward(q.cuda(), kk, vv, chunk_offsets=offs, kv_chunk_stride=stride, scale=scale,
                              n_splits=splits, block_m=128)
        torch.cuda.synchronize()
        check(out, lse, ref_out, ref_lse, f"forward D={D} Sq={Sq} lens={lens} padded={padded} splits={splits}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"Sq{c[0]}-" + "_".join(map(str, c[1])))
def test_key_groups_ring_steps(ra, D, case):
    """The ring's loop, one step per chunk (the Accum epilogue after the
    two groups' merge), against one-shot attention over all chunks."""
    Sq, lens = case
    B, H = 1, 2
    offs = [0]
    for n in lens:
        offs.append(offs[-1] + n)
    Skv = offs[-1]
    q, k, v = draw(2000 + Sq + Skv + D, B, Sq, Skv, H, D)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    ref_out, ref_lse = oracle.attention_fp64(f64(q), f64(k), f64(v), scale)
    print(f"case D={D} Sq={Sq} lens={lens}", flush=True)
    qd = q.cuda()
    out = torch.empty((B, Sq, H, D), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda:0")
    ra.acc_init(out, lse)
    for c in range(len(lens)):
        kc = k[:, offs[c]:offs[c + 1]].contiguous().cuda()
        vc = v[:, offs[c]:offs[c + 1]].contiguous().cuda()
        ra.step(qd, kc, vc, out, lse, scale=scale, n_splits=1, block_m=128)
    torch.cuda.synchronize()
    check(out, lse, ref_out, ref_lse, f"ring steps D={D} Sq={Sq} lens={lens}")
