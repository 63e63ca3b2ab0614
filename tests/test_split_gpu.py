"""K/V splits: ringattn_step_split (the ring step with its chunk's keys
spread over several workgroups per query tile, whose partials a merge kernel
combines into the float32 accumulator) and the reuse of one split workspace
across calls with different inputs.  Tolerances as in test_parity_gpu: max|dout| <= 1e-2,
max|dlse| <= 1e-3 against the fp64 oracle on the same bf16 inputs."""

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


@functools.lru_cache(maxsize=None)
def inputs(name):
    return W.make_inputs(name)


@functools.lru_cache(maxsize=None)
def reference(name):
    x = inputs(name)
    return oracle.attention_fp64(W.to_f64(x["q"]), W.to_f64(x["k"]), W.to_f64(x["v"]), x["scale"])


def check(out, lse, ref_out, ref_lse, what):
    o = out.detach().to("cpu", torch.float64).numpy()
    l = lse.detach().to("cpu", torch.float64).numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), f"{what}: non-finite result"
    eo, el = float(np.max(np.abs(o - ref_out))), float(np.max(np.abs(l - ref_lse)))
    print(f"{what}: max|dout|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= OUT_TOL and el <= LSE_TOL, f"{what}: out {eo}, lse {el}"


@pytest.mark.parametrize("name", ["tiny", "flux", "ring_anything"])
@pytest.mark.parametrize("splits,block_m", [(0, 0), (1, 256), (2, 256), (3, 256), (1, 128), (5, 128), (4, 128)])
def test_split_step_ring_loop(ra, name, splits, block_m):
    """The ring's loop with ringattn_step_split: one workspace serves every
    chunk; after the last chunk the accumulators hold the oracle's result.
    One split of 256 rows is the 8-wave kernel's in-place LSE merge into the
    accumulator (staged through LDS at D = 128), one of 128 rows the 4-wave
    kernel's; with ragged query rows (Ring Anything: 577) and, for tiny,
    D = 64."""
    x = inputs(name)
    w = x["workload"]
    print(f"case {name} splits={splits} block_m={block_m}", flush=True)
    offs = oracle.chunk_offsets(w.seq_len, w.n_chunks, w.ring_anything)
    q, k, v = x["q"].cuda(), x["k"].cuda(), x["v"].cuda()
    longest = max(offs[c + 1] - offs[c] for c in range(w.n_chunks))
    n_sp, bm, ws_bytes = ra.step_plan(tuple(q.shape), longest, splits, block_m)
    ws = ra.new_workspace(ws_bytes, q.device)
    out_acc, lse_acc = ra.new_accumulators(q)
    for c in range(w.n_chunks):
        kc = k[:, offs[c]:offs[c + 1]].contiguous()
        vc = v[:, offs[c]:offs[c + 1]].contiguous()
        ra.step(q, kc, vc, out_acc, lse_acc, scale=x["scale"], n_splits=n_sp, block_m=bm, workspace=ws)
    torch.cuda.synchronize()
    check(out_acc, lse_acc, *reference(name), f"split step {name} ({n_sp} splits, {bm} rows)")


def test_split_step_empty_chunk_and_planned_default(ra):
    """A split step into empty accumulators equals one-chunk attention, and a
    later empty chunk changes nothing."""
    x = inputs("ring_anything")
    w = x["workload"]
    q = x["q"].cuda()
    n_sp, bm, ws_bytes = ra.step_plan(tuple(q.shape), 577, 3, 256)
    assert (n_sp, bm) == (3, 256) and ws_bytes > 0
    out_acc, lse_acc = ra.new_accumulators(q)
    kc = x["k"][:, :577].contiguous().cuda()
    vc = x["v"][:, :577].contiguous().cuda()
    ra.step(q, kc, vc, out_acc, lse_acc, scale=x["scale"], n_splits=3, block_m=256)
    before = (out_acc.clone(), lse_acc.clone())
    empty = torch.empty((1, 0, w.heads, w.head_dim), dtype=torch.bfloat16, device="cuda:0")
    ra.step(q, empty, empty, out_acc, lse_acc, scale=x["scale"], n_splits=3)
    torch.cuda.synchronize()
    assert torch.equal(out_acc, before[0]) and torch.equal(lse_acc, before[1])
    ref_o, ref_l = oracle.attention_fp64(W.to_f64(x["q"]), W.to_f64(x["k"][:, :577]), W.to_f64(x["v"][:, :577]),
                                         x["scale"])
    check(out_acc, lse_acc, ref_o, ref_l, "split step, first chunk")


def test_split_forward_reuses_workspace_bitwise(ra):
    """Forward with splits, called five times on one workspace: every result
    is bit-identical."""
    x = inputs("flux")
    w = x["workload"]
    q, k, v = x["q"].cuda(), x["k"].cuda(), x["v"].cuda()
    offs = ra.chunk_offsets(w.seq_len, w.n_chunks)
    n_sp, bm, ws_bytes = ra.forward_plan(tuple(q.shape), offs, 4, 256)
    ws = ra.new_workspace(ws_bytes, q.device)
    results = []
    for _ in range(5):
        out, lse = ra.forward(q, k, v, chunk_offsets=offs, scale=x["scale"], n_splits=n_sp, block_m=bm, workspace=ws)
        results.append((out.clone(), lse.clone()))
    torch.cuda.synchronize()
    for o, l in results[1:]:
        assert torch.equal(o, results[0][0]) and torch.equal(l, results[0][1])
    check(*results[0], *reference("flux"), "forward, 4 splits, reused workspace")


def test_split_workspace_alternating_inputs(ra):
    """Two different shards alternate on one split workspace at a large grid
    (864 workgroups): every result equals that input's first result bit for
    bit, so no merge ever reads a partial left by the other input."""
    x = inputs("ulysses_even")
    q, k, v = x["q"].cuda(), x["k"].cuda(), x["v"].cuda()
    q2, v2 = q.flip(1).contiguous(), (-v).contiguous()
    offs = [0, k.shape[1]]
    n_sp, bm, ws_bytes = ra.forward_plan(tuple(q.shape), offs, 4, 128)
    assert n_sp == 4
    ws = ra.new_workspace(ws_bytes, q.device)
    first = {}
    for it in range(6):
        for tag, (qq, vv) in (("a", (q, v)), ("b", (q2, v2))):
            out, lse = ra.forward(qq, k, vv, chunk_offsets=offs, scale=x["scale"], n_splits=n_sp, block_m=bm,
                                  workspace=ws)
            if tag not in first:
                first[tag] = (out.clone(), lse.clone())
            else:
                assert torch.equal(out, first[tag][0]) and torch.equal(lse, first[tag][1]), f"call {it} input {tag}"
    torch.cuda.synchronize()
    assert not torch.equal(first["a"][0], first["b"][0])
    rows = [0, 1, 777, 4607]
    ref_o, ref_l = oracle.attention_rows_fp64(W.to_f64(x["q"]), W.to_f64(x["k"]), W.to_f64(x["v"]), x["scale"], rows)
    check(first["a"][0][:, rows], first["a"][1][:, :, rows], ref_o, ref_l, "alternating inputs, sampled rows")
