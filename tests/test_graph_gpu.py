"""The whole step (both map builds, the forward, both backward kernels)
captured in a HIP graph and replayed.  The library only launches kernels
(no allocation, memset or copy on the stream) and every counter a kernel
reads is reset by an earlier kernel of the same step, so a replay needs
nothing from the host: each replay's outputs must be bit-identical to the
eager step's, even with the maps and the workspace overwritten with garbage
and eager work in between."""
import pytest
import torch

import bench
from gpu_path import api, say
from workloads.generate import make_workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [5, 2])
def test_step_replays_bit_identically_in_a_graph(cfg):
    A = api()
    w = make_workload(cfg, 0)  # the group packs split key tiles, so their arrival counters run too
    q, k, v, do = (x.cuda().contiguous() for x in (w.q, w.k, w.v, w.do))
    r = bench.Runner(A, torch, w.packset, q, k, v, do, w.Hq, w.Hkv, w.D, w.scale)
    outs = lambda: (r.o, r.lse, r.dq, r.dk, r.dv)  # noqa: E731
    names = ("o", "lse", "dq", "dk", "dv")
    r.step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs()]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        r.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        r.step()
    torch.cuda.synchronize()

    for rep in range(4):
        # eager work between replays: garbage into every buffer the step writes
        for t in outs():
            t.fill_(float("nan"))
        for buf in (r.fmap.buffer, r.bmap.buffer, r.ws):
            buf.fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say("graph replay", cfg, rep)
        for name, want, got in zip(names, ref, outs()):
            assert torch.equal(want, got), (cfg, rep, name)
    # the eager step still agrees after the replays
    r.step()
    torch.cuda.synchronize()
    for name, want, got in zip(names, ref, outs()):
        assert torch.equal(want, got), (cfg, "eager", name)
