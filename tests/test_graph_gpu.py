"""The library's calls enqueue kernels on the caller's stream and nothing else
(no allocation, synchronisation or memset), so they can be captured in a HIP
graph: the whole shard with a K/V split (attention + split merge, caller
workspace) and the ring's own loop (accumulator initialisation + one step
per chunk).  Each graph is replayed several times with eager calls of the
same work in between, and every replay must equal the eager result bit for
bit (the kernels use no atomics, so repeated runs are deterministic).
"""

import pytest
import torch

from context_attention_diffusion_ringattn_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ra():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    import context_attention_diffusion_ringattn_amd as ra_mod
    ra_mod._lib.lib()
    return ra_mod


def capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up on a side stream, as graph capture requires
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_forward_with_split_in_a_graph(ra):
    x = W.make_inputs("ring_anything")
    w = x["workload"]
    dev = torch.device("cuda:0")
    q, k, v = x["q"].to(dev), x["k"].to(dev), x["v"].to(dev)
    offs = ra.chunk_offsets(w.seq_len, w.n_chunks, True)
    n_splits, block_m, ws_bytes = ra.forward_plan(tuple(q.shape), offs, 3, 256)
    assert n_splits == 3 and ws_bytes > 0
    ws = ra.new_workspace(ws_bytes, dev)
    out = torch.empty((1, q.shape[1], w.heads, w.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((1, w.heads, q.shape[1]), dtype=torch.float32, device=dev)

    def run():
        ra.forward(q, k, v, chunk_offsets=offs, scale=x["scale"], n_splits=n_splits, block_m=block_m, out=out,
                   lse=lse, workspace=ws)

    run()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    g = capture(run)
    for rep in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {rep}"
        run()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"eager after replay {rep}"


def test_ring_loop_in_a_graph(ra):
    x = W.make_inputs("flux")
    w = x["workload"]
    dev = torch.device("cuda:0")
    q, k, v = x["q"].to(dev), x["k"].to(dev), x["v"].to(dev)
    offs = ra.chunk_offsets(w.seq_len, w.n_chunks, False)
    chunks = [(k[:, offs[c]:offs[c + 1]].contiguous(), v[:, offs[c]:offs[c + 1]].contiguous())
              for c in range(w.n_chunks)]
    o_acc = torch.empty((1, q.shape[1], w.heads, w.head_dim), dtype=torch.float32, device=dev)
    l_acc = torch.empty((1, w.heads, q.shape[1]), dtype=torch.float32, device=dev)

    def run():
        ra.acc_init(o_acc, l_acc)
        for kc, vc in chunks:
            ra.step(q, kc, vc, o_acc, l_acc, scale=x["scale"])

    run()
    torch.cuda.synchronize()
    ref_o, ref_l = o_acc.clone(), l_acc.clone()
    g = capture(run)
    for rep in range(4):
        o_acc.fill_(123.0)
        l_acc.fill_(123.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_acc, ref_o) and torch.equal(l_acc, ref_l), f"replay {rep}"
        run()
        torch.cuda.synchronize()
        assert torch.equal(o_acc, ref_o) and torch.equal(l_acc, ref_l), f"eager after replay {rep}"
