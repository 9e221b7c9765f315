"""The ways bench.py runs the kernels besides the plain step.  The dense-map
baseline (every tile pair visited as a partial tile, so the kernels evaluate
the mask everywhere, including tiles where it removes every pair) against
the oracle: the baseline the sparse path is compared with must compute the
same attention, and it drives the masked code paths through tiles that the
sparse map would skip.  The backward's two stages run one at a time, as
bench.py times them."""
import numpy as np
import pytest
import torch

import bench
import oracle
from gpu_path import api, rel_l2, say
from workloads.generate import Pack, PackSet, descriptor_arrays, make_workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("heads", [(8, 2, 128), (3, 1, 64)])
def test_dense_map_baseline_matches_the_oracle(heads):
    A = api()
    ps = PackSet(2, 300, [Pack(0, 0, 60, (50, 70)), Pack(0, 190, 10, (40, 3)), Pack(1, 9, 0, (100, 120))])
    w = make_workload(None, 4, packset=ps, heads=heads)
    q, k, v, do = (x.cuda().contiguous() for x in (w.q, w.k, w.v, w.do))
    r = bench.Runner(A, torch, ps, q, k, v, do, w.Hq, w.Hkv, w.D, w.scale, dense=True)
    r.step()
    torch.cuda.synchronize()
    assert int(r.fmap.q2k_cnt()[:, :, 0].sum()) == 0            # no tile left full
    assert int(r.fmap.q2k_cnt()[:, :, 1].sum()) == ps.B * r.fmap.nqt * r.fmap.nkt
    P, R = descriptor_arrays(ps)
    pk, br, _ = oracle.token_ids(P, R, ps.B, ps.S)
    m = oracle.attention_mask(pk, br)
    O, L = oracle.attn_fwd(w.q, w.k, w.v, m, w.scale)
    dq, dk, dv = oracle.attn_bwd(w.q, w.k, w.v, w.do, m, w.scale)
    valid = torch.from_numpy(pk >= 0)
    vl = valid[:, None, :].expand(ps.B, w.Hq, ps.S)
    errs = {"o": rel_l2(r.o.cpu()[valid], O[valid])}
    for name, x, ref in (("dq", r.dq, dq), ("dk", r.dk, dk), ("dv", r.dv, dv)):
        errs[name] = rel_l2(x.cpu()[valid], ref[valid])
        assert (x.cpu()[~valid] == 0).all(), name
    lse = r.lse.cpu().double()
    say("dense map", heads, errs)
    assert max(errs.values()) <= 1e-2, errs
    assert float((lse[vl] - L[vl]).abs().max()) <= 1e-3
    assert torch.isneginf(lse[~vl]).all() and (r.o.cpu()[~valid] == 0).all()


def test_backward_stages_one_at_a_time_equal_the_whole_backward():
    """pba_packed_attn_bwd_stages with the dQ stage, then the dK/dV stage
    (the way bench.py times them) gives bit-identical gradients to one call
    with both stages."""
    A = api()
    w = make_workload(5, 0)  # the group packs: split key tiles included
    q, k, v, do = (x.cuda().contiguous() for x in (w.q, w.k, w.v, w.do))
    r = bench.Runner(A, torch, w.packset, q, k, v, do, w.Hq, w.Hkv, w.D, w.scale)
    r.build_maps()
    r.fwd()
    r.bwd(A.BWD_ALL)
    torch.cuda.synchronize()
    whole = [t.clone() for t in (r.dq, r.dk, r.dv)]
    for t in (r.dq, r.dk, r.dv):
        t.fill_(float("nan"))
    r.bwd(A.BWD_DQ)
    r.bwd(A.BWD_DKDV)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), whole, (r.dq, r.dk, r.dv)):
        assert torch.equal(a, b), name
