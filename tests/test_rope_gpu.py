"""GPU rotary embedding at packed positions vs the oracle (fp64).

Tolerance, per element: the output is rounded to bf16 (half an ulp,
2^-9 relative) and the angle pos * base^(-2i/D) is formed in fp32 (relative
error about 2^-22, i.e. at most 2.5e-3 rad for positions below 10^4), so
|y - y_ref| <= 2^-8 |y_ref| + 3e-3 (|x_i| + |x_{i+D/2}|)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import rope as R
from gpu_path import api, build_map, say
from workloads.generate import Pack, PackSet, descriptor_arrays, make_packset, random_packset

pytestmark = pytest.mark.gpu


def _bound_ok(x, y, yref, rel=2.0 ** -8):
    D = x.shape[-1]
    xs = x.abs()
    pair = torch.cat([xs[..., : D // 2] + xs[..., D // 2:]] * 2, dim=-1)
    return bool(((y - yref).abs() <= rel * yref.abs() + 3e-3 * pair).all())


def _same_rotation(x, y1, y2):
    """Two bf16 roundings of (nearly) the same rotation differ by at most one
    bf16 ulp (2^-7 relative) plus the fp32 angle error of each."""
    return _bound_ok(x, y1, y2, rel=2.0 ** -7)


def _run(ps, H, D, base, seed, inverse=False, in_place=False):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((ps.B, ps.S, H, D), generator=g).to(torch.bfloat16)
    m = build_map(ps, 64, 64)
    A = api()
    xd = x.cuda()
    y = A.packed_rope(m, xd, base, inverse, out=xd if in_place else None)
    torch.cuda.synchronize()
    P, Rl = descriptor_arrays(ps)
    pos, _, _, _ = oracle.positions(P, Rl, ps.B, ps.S)
    yref = R.packed_rope(x.double(), pos, base, inverse)
    return x.double(), y.cpu().double(), yref


@pytest.mark.parametrize("cfg,H,D", [(1, 2, 64), (2, 32, 128), (2, 8, 128), (5, 8, 128)])
def test_workloads(cfg, H, D):
    ps = make_packset(cfg)
    say("rope", cfg, H, D, ps.B, ps.S)
    x, y, yref = _run(ps, H, D, 1e6, cfg)
    assert _bound_ok(x, y, yref)


@pytest.mark.parametrize("seed", range(4))
def test_random_ragged_inverse_and_in_place(seed):
    rng = np.random.default_rng(900 + seed)
    ps = random_packset(rng, B=int(rng.integers(1, 4)), S=int(rng.integers(1, 500)), max_packs_per_row=4,
                        max_resp=4, max_len=int(rng.integers(2, 150)))
    D = (64, 128)[seed % 2]
    H = int(rng.integers(1, 7))
    say("rope random", seed, ps.B, ps.S, H, D)
    x, y, yref = _run(ps, H, D, 10000.0, seed, inverse=bool(seed & 1), in_place=seed >= 2)
    assert _bound_ok(x, y, yref)


def test_pad_is_identity_and_round_trip():
    ps = make_packset(2)
    A = api()
    m = build_map(ps, 64, 64)
    g = torch.Generator().manual_seed(3)
    x = torch.randn((ps.B, ps.S, 8, 128), generator=g).to(torch.bfloat16).cuda()
    y = A.packed_rope(m, x, 1e6)
    z = A.packed_rope(m, y, 1e6, inverse=True)
    torch.cuda.synchronize()
    P, Rl = descriptor_arrays(ps)
    pk = oracle.token_ids(P, Rl, ps.B, ps.S)[0]
    pad = torch.from_numpy(pk < 0)
    assert torch.equal(y.cpu()[pad], x.cpu()[pad])
    # forward then inverse: back to x up to two bf16 roundings
    err = (z.float() - x.float()).abs()
    assert bool((err <= 2.0 ** -7 * x.float().abs() + 2e-2).all())


def test_invalid_map_writes_nothing():
    A = api()
    ps = make_packset(1)
    P, Rl = descriptor_arrays(ps)
    P = P.copy()
    P[0, 0] = 5  # row outside [0, B)
    pd, rd = A.descriptors_to_device(P, Rl)
    m = A.pack_block_map(pd, rd, ps.B, ps.S, 64, 64)
    x = torch.ones((ps.B, ps.S, 2, 64), dtype=torch.bfloat16, device="cuda")
    y = torch.full_like(x, 7.0)
    A.packed_rope(m, x, 1e4, out=y)
    torch.cuda.synchronize()
    assert (y == 7.0).all()


def test_packed_rope_attention_equals_pairwise():
    """Content vectors -> pba_packed_rope -> packed forward equals, on every
    response row, causal attention over that response's own [prompt |
    response] sequence rotated at positions 0..n-1 (the oracle), for the
    Qwen3-8B-shaped packs at reduced width (the property aligned positions
    exist for: "DPO Preference Packing", section "Layout requirements")."""
    from workloads.generate import make_workload
    A = api()
    w = make_workload(2, 0)
    ps = w.packset
    H, D = 4, 128
    g = torch.Generator().manual_seed(11)
    xq, xk, xv = (torch.randn((ps.B, ps.S, H, D), generator=g) for _ in range(3))
    xq, xk, xv = (t.to(torch.bfloat16) for t in (xq, xk, xv))
    fm = build_map(ps, *A.fwd_tile(H, H, D))
    q = A.packed_rope(fm, xq.cuda(), 1e6)
    k = A.packed_rope(fm, xk.cuda(), 1e6)
    o, lse = A.packed_attn_fwd(fm, q, k, xv.cuda().contiguous(), 1.0 / 128 ** 0.5)
    torch.cuda.synchronize()
    o = o.cpu().double()
    say("rope + attention vs pairwise", ps.B, ps.S)
    for pk in ps.packs:
        prompt = list(range(pk.start, pk.start + pk.prompt_len))
        at = pk.start + pk.prompt_len
        for r in pk.resp_lens:
            rows = prompt + list(range(at, at + r))
            at += r
            n = len(rows)
            qq = R.rope(xq[pk.row, rows].double(), list(range(n)), 1e6)[None]
            kk = R.rope(xk[pk.row, rows].double(), list(range(n)), 1e6)[None]
            vv = xv[pk.row, rows].double()[None]
            O, _ = oracle.attn_fwd(qq, kk, vv, np.tril(np.ones((1, n, n), dtype=bool)), 1.0 / 128 ** 0.5)
            got = o[pk.row, rows[len(prompt):]]
            ref = O[0, len(prompt):]
            assert float((got - ref).abs().max()) <= 2e-2, float((got - ref).abs().max())


def _rope_case(w, base):
    """GPU: rotate Q, K at the packed positions, forward, fused-rotation
    backward.  Oracle inputs: the same bf16 Q, K, V, dO."""
    A = api()
    ps = w.packset
    q, k, v, do = (x.cuda().contiguous() for x in (w.q, w.k, w.v, w.do))
    fm = build_map(ps, *A.fwd_tile(w.Hq, w.Hkv, w.D))
    bm = build_map(ps, *A.bwd_tile(w.Hq, w.Hkv, w.D))
    kr = A.packed_rope(fm, k, base)
    # fused: Q rotated inside the forward (which also writes it), gradients
    # rotated back inside the backward
    o, lse, qr = A.packed_attn_fwd_rope(fm, q, kr, v, base, w.scale)
    dq, dk, dv = A.packed_attn_bwd_rope(fm, bm, qr, kr, v, o, lse, do, base, w.scale)
    # unfused: rotation passes around the plain forward and backward
    qr_u = A.packed_rope(fm, q, base)
    o_u, lse_u = A.packed_attn_fwd(fm, qr_u, kr, v, w.scale)
    dq_r, dk_r, dv_u = A.packed_attn_bwd(fm, bm, qr_u, kr, v, o_u, lse_u, do, w.scale)
    dq_u, dk_u = A.packed_rope(fm, dq_r, base, inverse=True), A.packed_rope(fm, dk_r, base, inverse=True)
    torch.cuda.synchronize()
    P, Rl = descriptor_arrays(ps)
    pos = oracle.positions(P, Rl, ps.B, ps.S)[0]
    return {"o": o.cpu(), "dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu(), "o_u": o_u.cpu(), "dq_u": dq_u.cpu(),
            "dk_u": dk_u.cpu(), "dv_u": dv_u.cpu(), "qr": qr.cpu(), "qr_u": qr_u.cpu(), "q": w.q, "pos": pos, "P": P,
            "R": Rl}


def _rel(x, ref):
    x, ref = x.double(), ref.double()
    return float((x - ref).norm() / ref.norm())


def test_fused_rope_backward_tiny_vs_oracle():
    from workloads.generate import make_workload
    w = make_workload(1, 0, unscaled=True)
    base = 1e4
    got = _rope_case(w, base)
    ps = w.packset
    pk, br, _ = oracle.token_ids(got["P"], got["R"], ps.B, ps.S)
    mask = oracle.attention_mask(pk, br)
    qr, kr = R.packed_rope(w.q, got["pos"], base), R.packed_rope(w.k, got["pos"], base)
    O, _ = oracle.attn_fwd(qr, kr, w.v, mask, w.scale)
    dqr, dkr, dv = oracle.attn_bwd(qr, kr, w.v, w.do, mask, w.scale)
    dq, dk = R.packed_rope(dqr, got["pos"], base, inverse=True), R.packed_rope(dkr, got["pos"], base, inverse=True)
    say("fused rope bwd tiny", _rel(got["dq"], dq), _rel(got["dk"], dk), _rel(got["dv"], dv))
    assert _rel(got["o"], O) <= 1e-2 and _rel(got["o_u"], O) <= 1e-2
    # the forward's rotated Q equals the rotation pass's up to bf16 rounding
    assert _same_rotation(got["q"].double(), got["qr"].double(), got["qr_u"].double())
    for name, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert _rel(got[name], ref) <= 1e-2, name
        assert _rel(got[name + "_u"], ref) <= 1e-2, name + " unfused"


def test_fused_rope_backward_qwen3_packs_sampled():
    from workloads.generate import make_workload
    w = make_workload(2, 0, unscaled=True)
    base = 1e6
    got = _rope_case(w, base)
    ps = w.packset
    pk, br, _ = oracle.token_ids(got["P"], got["R"], ps.B, ps.S)
    rng = np.random.default_rng(5)
    b, g = int(rng.integers(0, ps.B)), int(rng.integers(0, w.Hkv))
    valid = np.nonzero(pk[b] >= 0)[0]
    qrows = np.sort(rng.choice(valid, size=64, replace=False))
    krows = np.sort(rng.choice(valid, size=64, replace=False))
    mb = oracle.attention_mask(pk, br, row=b)
    qr, kr = R.packed_rope(w.q, got["pos"], base), R.packed_rope(w.k, got["pos"], base)
    dqs, dks, dvs = oracle.attn_bwd_sampled(qr, kr, w.v, w.do, mb, b, g, qrows, krows, w.scale)
    G = w.Hq // w.Hkv
    pos_b = got["pos"][b]
    dq_ref = R.rope(dqs.permute(1, 0, 2), pos_b[qrows], base, inverse=True).permute(1, 0, 2)  # [G, n, D]
    dk_ref = R.rope(dks[:, None], pos_b[krows], base, inverse=True)[:, 0]
    dq = torch.stack([got["dq"][b, qrows, h] for h in range(g * G, (g + 1) * G)])
    e = (_rel(dq, dq_ref), _rel(got["dk"][b, krows, g], dk_ref), _rel(got["dv"][b, krows, g], dvs))
    say("fused rope bwd qwen3 packs sampled", b, g, e)
    assert max(e) <= 1e-2, e
    # forward: sampled rows of one head against the oracle on rotated inputs
    h = g * G
    Os, _ = oracle.attn_fwd_rows(qr, kr, w.v, mb, b, h, qrows, w.scale)
    assert _rel(got["o"][b, qrows, h], Os) <= 1e-2
    assert _same_rotation(got["q"].double(), got["qr"].double(), got["qr_u"].double())


@pytest.mark.parametrize("heads", [(4, 2, 128), (12, 2, 128), (8, 1, 64), (8, 2, 64), (8, 2, 128), (2, 2, 128),
                                   (3, 1, 64)])
def test_fused_rope_variants_vs_oracle(heads):
    """The fused-rotation forward and backward of every compiled variant (q
    heads per workgroup 4, 2 and 1 at D = 64 and 128) against the oracle on
    random ragged packs: O on rotated inputs, dQ and dK rotated back to the
    unrotated Q and K, dV; whole tensors, every valid element."""
    rng = np.random.default_rng(4200 + 7 * heads[0] + heads[2])
    ps = random_packset(rng, B=2, S=int(rng.integers(150, 400)), max_packs_per_row=3, max_resp=3, max_len=110)
    if not ps.packs:
        ps = make_packset(1)
    say("fused rope variant", heads, ps.B, ps.S, len(ps.packs))
    _rope_vs_oracle(ps, heads)


# Short and degenerate layouts: a pack with an empty prompt and two empty
# branches beside an all-pad row; an empty first response; a prompt-only
# pack, an empty pack and 40 one-token responses; rows ending inside the
# first tile, one holding a single token at its last position.
ROPE_EDGE_LAYOUTS = [
    PackSet(2, 70, [Pack(1, 0, 0, (0, 0, 70))]),
    PackSet(1, 130, [Pack(0, 0, 64, (0, 66))]),
    PackSet(1, 200, [Pack(0, 3, 5, ()), Pack(0, 8, 0, ()), Pack(0, 8, 0, (1,) * 40)]),
    PackSet(2, 17, [Pack(0, 0, 3, (7, 7)), Pack(1, 16, 1, ())]),
]


@pytest.mark.parametrize("case", range(len(ROPE_EDGE_LAYOUTS)))
def test_fused_rope_edge_layouts(case):
    ps = ROPE_EDGE_LAYOUTS[case]
    say("fused rope edge", case, ps.B, ps.S, len(ps.packs))
    _rope_vs_oracle(ps, (4, 2, 128))


def _rope_vs_oracle(ps, heads):
    from workloads.generate import make_workload
    w = make_workload(None, 6, packset=ps, heads=heads, unscaled=True)
    base = 1e4
    got = _rope_case(w, base)
    pk, br, _ = oracle.token_ids(got["P"], got["R"], ps.B, ps.S)
    mask = oracle.attention_mask(pk, br)
    qr, kr = R.packed_rope(w.q, got["pos"], base), R.packed_rope(w.k, got["pos"], base)
    O, L = oracle.attn_fwd(qr, kr, w.v, mask, w.scale)
    dqr, dkr, dv = oracle.attn_bwd(qr, kr, w.v, w.do, mask, w.scale)
    dq, dk = R.packed_rope(dqr, got["pos"], base, inverse=True), R.packed_rope(dkr, got["pos"], base, inverse=True)
    valid = torch.from_numpy(pk >= 0)
    o = got["o"].double()
    assert float((o - O).abs()[valid].max()) <= 1e-2
    errs = {"o": _rel(got["o"][valid], O[valid])}
    for name, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
        errs[name] = _rel(got[name][valid], ref[valid])
        assert (got[name][~valid] == 0).all(), name
    say("  rel-L2", errs)
    assert max(errs.values()) <= 1e-2, errs
    assert _same_rotation(got["q"].double(), got["qr"].double(), got["qr_u"].double())
