"""pba_packed_attn_bwd_noalloc (the library's own device scratch, no
workspace argument) against pba_packed_attn_bwd on the same inputs, called
through the C ABI: three calls in a row on one device, each on a smaller
input than the one before (group packs with split key tiles, the
Qwen3-8B-shaped packs, the tiny pack), so every call finds the scratch as
the previous, larger call left it.  Each result is bit-identical to the
workspace entry point's (every split pair fits the scratch at these sizes)
and, a fortiori, within the oracle's gradient bar of it."""
import ctypes

import pytest
import torch

from gpu_path import api, build_map, rel_l2, say
from workloads.generate import make_workload

pytestmark = pytest.mark.gpu

G_REL = 1e-2


def _noalloc_matches(cfg):
    A = api()
    w = make_workload(cfg)
    say("no-alloc backward", cfg, w.packset.B, w.packset.S, w.Hq, w.Hkv, w.D)
    q, k, v, do = (x.cuda().contiguous() for x in (w.q, w.k, w.v, w.do))
    fm = build_map(w.packset, *A.fwd_tile(w.Hq, w.Hkv, w.D))
    bm = build_map(w.packset, *A.bwd_tile(w.Hq, w.Hkv, w.D))
    o, lse = A.packed_attn_fwd(fm, q, k, v, w.scale)
    ref = A.packed_attn_bwd(fm, bm, q, k, v, o, lse, do, w.scale)
    outs = [torch.full_like(x, 3.0) for x in (q, k, v)]
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    rc = A._lib.pba_packed_attn_bwd_noalloc(ctypes.byref(fm.struct), ctypes.byref(bm.struct), q.data_ptr(),
                                            k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                                            outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(), B, S, Hq, Hkv,
                                            D, w.scale, int(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, A.strerror(rc)
    torch.cuda.synchronize()
    for name, x, y in zip(("dq", "dk", "dv"), outs, ref):
        e = rel_l2(x.cpu(), y.cpu())
        say("  ", name, "rel-L2 vs workspace entry", e, "bit-identical", torch.equal(x, y))
        assert e <= G_REL, (cfg, name, e)
        assert torch.equal(x, y), (cfg, name)


def test_noalloc_matches_workspace_entry_on_shrinking_inputs():
    for cfg in (5, 2, 1):
        _noalloc_matches(cfg)
