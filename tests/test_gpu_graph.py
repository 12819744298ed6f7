"""fsa_bounds + fsa_attention captured in a HIP graph (needs an MI355X).

The library allocates nothing and clears its accumulators with its own kernels
(no memset nodes), so one step of the path can be captured and replayed. Each
replay must give exactly the eager result: the graph is replayed several
times, with eager work and a refill of the outputs between replays.
"""
import sys

import pytest
import torch

import synthetic

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("center", [False, True], ids=["plain", "centred"])
def test_graph_replays_equal_eager(center):
    import frame_windowed_block_amd as fsa
    fsa.lib()
    wl = synthetic.Workload("graph", 1, 2, 128, 3, 1200, 1, 0, dist="key_offset" if center else "normal",
                            seed=21)
    _say(f"graph capture: F={wl.frames} T={wl.tokens_per_frame} H={wl.heads} centred={center}")
    q, k, v = (x.cuda() for x in synthetic.make_inputs(wl))
    dplan = fsa.DevicePlan(wl.frames, wl.tokens_per_frame, wl.window, wl.ref_frame)
    info = dplan.info
    qn = torch.empty((1, wl.heads, wl.seq_len), dtype=torch.float32, device="cuda")
    km = torch.empty((1, wl.heads, info.n_kblocks), dtype=torch.float32, device="cuda")
    el = torch.empty((1, wl.heads), dtype=torch.int32, device="cuda")
    bm = torch.empty((1, wl.heads), dtype=torch.float32, device="cuda")
    mu = torch.empty((1, wl.heads, wl.head_dim), dtype=torch.float32, device="cuda") if center else None
    o = torch.empty_like(q)

    def run():
        fsa.bounds(dplan, q, k, wl.scale, 0.0, 0, 0, qn, km, el, bm, kmean=mu)
        fsa.attention(dplan, q, k, v, qn, km, el, wl.scale, 0, 0, out=o, kmean=mu)

    run()
    torch.cuda.synchronize()
    o_ref, el_ref, bm_ref = o.clone(), el.clone(), bm.clone()
    assert int(el_ref.sum()) == wl.heads            # both heads on the bound path

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()                                       # warm-up on the capture stream's side
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()

    for r in range(4):
        o.fill_(-3.0)
        el.fill_(-1)
        bm.fill_(-1.0)
        torch.cuda.synchronize()
        _ = (q.float() * 2.0).sum().item()          # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"replay {r}: output differs from the eager run"
        assert torch.equal(el, el_ref) and torch.equal(bm, bm_ref), f"replay {r}: bounds differ"
    _say(f"graph capture: {r + 1} replays equal to the eager run")
