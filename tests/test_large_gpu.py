"""Maximum-size parity: a packed key range of 2^24 + 37 keys (K and V of
4.3 GB each, so tile addresses pass 2^32 bytes) against the oracle on
sampled query rows.  K/V are drawn on the device from a seeded generator;
the oracle streams them back chunk by chunk and combines the fp64 chunk
partials with its own LSE merge (exact up to fp64 rounding, pinned in the
oracle tests).  Tolerances as everywhere: 1e-2 on out, 1e-3 on the LSE."""

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ra():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    import context_attention_diffusion_ringattn_amd as ra_mod
    ra_mod._lib.lib()
    return ra_mod


def test_sixteen_million_keys(ra):
    B, H, D, Sq = 1, 1, 128, 300
    S = (1 << 24) + 37
    print(f"case large: Sq={Sq} Skv={S} H={H} D={D}", flush=True)
    g = torch.Generator(device="cuda:0").manual_seed(1234)
    q = torch.randn((B, Sq, H, D), generator=g, device="cuda:0", dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn((B, S, H, D), generator=g, device="cuda:0", dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((B, S, H, D), generator=g, device="cuda:0", dtype=torch.float32).to(torch.bfloat16)
    scale = ra.default_scale(D)
    out, lse = ra.forward(q, k, v, chunk_offsets=[0, S], scale=scale)
    torch.cuda.synchronize()
    rows = [0, 1, 137, 255, 256, 299]
    q64 = q[:, rows].double().cpu().numpy()
    acc_o = np.zeros((B, len(rows), H, D))
    acc_l = np.full((B, H, len(rows)), -np.inf)
    step = 1 << 21
    for lo in range(0, S, step):
        hi = min(S, lo + step)
        kc = k[:, lo:hi].double().cpu().numpy()
        vc = v[:, lo:hi].double().cpu().numpy()
        po, pl = oracle.chunk_partial_fp64(q64, kc, vc, scale)
        acc_o, acc_l = oracle.lse_merge_fp64(acc_o, acc_l, po, pl)
    go = out[:, rows].double().cpu().numpy()
    gl = lse[:, :, rows].double().cpu().numpy()
    eo, el = float(np.max(np.abs(go - acc_o))), float(np.max(np.abs(gl - acc_l)))
    print(f"large: max|dout|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert np.all(np.isfinite(go)) and eo <= 1e-2 and el <= 1e-3
