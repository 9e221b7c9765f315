"""Pins of the oracle's forward and backward (CPU only, float64)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle_pins import descriptors, rope
from workloads.generate import Pack, PackSet, make_workload

F64 = torch.float64


def _mask(B, S, pl):
    P, R = descriptors(pl)
    pk, br, st = oracle.token_ids(P, R, B, S)
    assert tuple(st) == (0, -1)
    return oracle.attention_mask(pk, br)


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=F64)


def test_rows_sum_to_one_and_lse():
    w = make_workload(1)
    m = _mask(1, 144, [(0, 0, 64, (32, 48))])
    ones = torch.ones_like(w.v, dtype=F64)
    O, L = oracle.attn_fwd(w.q, w.k, ones, m, w.scale)
    assert torch.allclose(O, torch.ones_like(O), rtol=0, atol=1e-12)
    q, k = w.q.to(F64), w.k.to(F64)
    for h in range(2):
        s = (q[0, :, h] @ k[0, :, h].T) * w.scale
        lse = torch.logsumexp(s.masked_fill(~torch.from_numpy(m[0]), float("-inf")), dim=1)
        assert torch.allclose(L[0, h], lse, rtol=0, atol=1e-12)


def test_pad_rows_are_zero_and_neg_inf():
    pl = [(0, 1, 3, (2,))]
    S = 9
    m = _mask(1, S, pl)
    q, k, v, do = (_rand((1, S, 2, 8), i) for i in range(4))
    O, L = oracle.attn_fwd(q, k, v, m, 0.3)
    pad = [0, 6, 7, 8]
    assert (O[0, pad] == 0).all() and torch.isinf(L[0][:, pad]).all() and (L[0][:, pad] < 0).all()
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, m, 0.3)
    assert (dq[0, pad] == 0).all() and (dk[0, pad] == 0).all() and (dv[0, pad] == 0).all()


@pytest.mark.parametrize("pl,S", [
    ([(0, 0, 0, (20,))], 20),          # zero-length prompt, one response: a plain causal document
    ([(0, 0, 17, ())], 17),            # prompt only
])
def test_single_sequence_equals_sdpa(pl, S):
    m = _mask(1, S, pl)
    q, k, v = (_rand((1, S, 4, 16), 10 + i) for i in range(3))
    O, _ = oracle.attn_fwd(q, k, v, m, 0.25)
    ref = F.scaled_dot_product_attention(q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2),
                                         is_causal=True, scale=0.25).transpose(1, 2)
    assert torch.allclose(O, ref, rtol=0, atol=1e-12)


def test_multi_document_row_equals_per_document_sdpa():
    """cu_seqlens-style rows: each pack alone is a causal document (p3, p5)."""
    pl = [(0, 0, 0, (5,)), (0, 5, 7, ()), (0, 14, 0, (9,))]
    S = 25
    m = _mask(1, S, pl)
    q, k, v = (_rand((1, S, 2, 8), 20 + i) for i in range(3))
    O, _ = oracle.attn_fwd(q, k, v, m, 0.5)
    for a, n in ((0, 5), (5, 7), (14, 9)):
        sl = slice(a, a + n)
        ref = F.scaled_dot_product_attention(q[:, sl].transpose(1, 2), k[:, sl].transpose(1, 2),
                                             v[:, sl].transpose(1, 2), is_causal=True, scale=0.5).transpose(1, 2)
        assert torch.allclose(O[:, sl], ref, rtol=0, atol=1e-12)


def _packed_vs_pairwise_setup(p=6, rls=(4, 5, 3), H=2, D=8, seed=0, positions="aligned"):
    """Content vectors -> RoPE at branch-aligned positions (prompt 0..p-1, each
    response p..p+r-1, p1 "Layout requirements": aligned positions)."""
    T = p + sum(rls)
    xq, xk, xv, xdo = (_rand((T, H, D), seed + i) for i in range(4))
    if positions == "aligned":
        pos = list(range(p))
        for r in rls:
            pos += list(range(p, p + r))
    else:  # naive sequential positions over the packed row
        pos = list(range(T))
    q = rope(xq, pos)[None]
    k = rope(xk, pos)[None]
    return xq, xk, xv, xdo, q, k, xv[None], xdo[None], T


def _pair_rows(p, rls, kk):
    start = p + sum(rls[:kk])
    return list(range(p)) + list(range(start, start + rls[kk]))


@pytest.mark.parametrize("positions,mask_kind,should_match", [
    ("aligned", "branch", True),
    ("sequential", "branch", False),   # negative control: naive positions
    ("aligned", "causal", False),      # negative control: plain causal mask
])
def test_packed_equals_pairwise(positions, mask_kind, should_match):
    p, rls, H, D, scale = 6, (4, 5, 3), 2, 8, 0.35
    xq, xk, xv, xdo, q, k, v, do, T = _packed_vs_pairwise_setup(p, rls, H, D, positions=positions)
    if mask_kind == "branch":
        m = _mask(1, T, [(0, 0, p, rls)])
    else:
        m = np.tril(np.ones((1, T, T), dtype=bool))
    O, L = oracle.attn_fwd(q, k, v, m, scale)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, m, scale)
    ok = True
    for kk in range(len(rls)):
        rows = _pair_rows(p, rls, kk)
        n = len(rows)
        pos = list(range(n))
        pq, pk_ = rope(xq[rows], pos)[None], rope(xk[rows], pos)[None]
        pv, pdo = xv[rows][None], xdo[rows][None]
        mc = np.tril(np.ones((1, n, n), dtype=bool))
        Op, Lp = oracle.attn_fwd(pq, pk_, pv, mc, scale)
        ok &= torch.allclose(O[0, rows], Op[0], rtol=1e-12, atol=1e-12)
        ok &= torch.allclose(L[0][:, rows], Lp[0], rtol=1e-12, atol=1e-12)
        # gradients of the response rows (their own dQ, and dK/dV of keys only
        # this branch sees) equal the pairwise copy's
        dqp, dkp, dvp = oracle.attn_bwd(pq, pk_, pv, pdo, mc, scale)
        resp = rows[p:]
        # pairwise dq is w.r.t. the rotated q; the packed q is rotated by the same angles on these rows
        ok &= torch.allclose(dq[0, resp], dqp[0, p:], rtol=1e-10, atol=1e-12)
        ok &= torch.allclose(dk[0, resp], dkp[0, p:], rtol=1e-10, atol=1e-12)
        ok &= torch.allclose(dv[0, resp], dvp[0, p:], rtol=1e-10, atol=1e-12)
    assert bool(ok) == should_match


def test_prompt_dkdv_is_sum_over_branches():
    """dK/dV of prompt keys in the packed row = sum of the pairwise rows'
    prompt dK/dV, with the prompt rows' dO counted once (backward is linear
    in dO): pair 1 carries dO on its prompt rows, the others carry zero."""
    p, rls, H, D, scale = 5, (3, 4, 2), 2, 8, 0.4
    xq, xk, xv, xdo, q, k, v, do, T = _packed_vs_pairwise_setup(p, rls, H, D, seed=7)
    m = _mask(1, T, [(0, 0, p, rls)])
    _, dk, dv = oracle.attn_bwd(q, k, v, do, m, scale)
    sk = torch.zeros((p, H, D), dtype=F64)
    sv = torch.zeros((p, H, D), dtype=F64)
    for kk in range(len(rls)):
        rows = _pair_rows(p, rls, kk)
        n = len(rows)
        pos = list(range(n))
        pq, pk_ = rope(xq[rows], pos)[None], rope(xk[rows], pos)[None]
        pdo = xdo[rows][None].clone()
        if kk > 0:
            pdo[0, :p] = 0
        _, dkp, dvp = oracle.attn_bwd(pq, pk_, xv[rows][None], pdo, np.tril(np.ones((1, n, n), dtype=bool)), scale)
        sk += dkp[0, :p]
        sv += dvp[0, :p]
    assert torch.allclose(dk[0, :p], sk, rtol=1e-10, atol=1e-12)
    assert torch.allclose(dv[0, :p], sv, rtol=1e-10, atol=1e-12)
    # in-layout form: runs with dO restricted to one branch's rows add up
    parts = [list(range(p))]
    off = p
    for r in rls:
        parts.append(list(range(off, off + r)))
        off += r
    acc = [torch.zeros_like(x) for x in (q, k, v)]
    for rows in parts:
        dsub = torch.zeros_like(do)
        dsub[0, rows] = do[0, rows]
        for a, g in zip(acc, oracle.attn_bwd(q, k, v, dsub, m, scale)):
            a += g
    full = oracle.attn_bwd(q, k, v, do, m, scale)
    for a, g in zip(acc, full):
        assert torch.allclose(a, g, rtol=1e-10, atol=1e-12)


def _loss(q, k, v, do, m, scale):
    O, _ = oracle.attn_fwd(q, k, v, m, scale)
    return float((O * do).sum())


def test_finite_differences():
    pl = [(0, 0, 4, (3, 5)), (0, 12, 2, (2,)), (0, 17, 0, (3,))]
    S, Hq, Hkv, D, scale = 22, 4, 2, 8, 0.37
    m = _mask(1, S, pl)
    q, k, v, do = _rand((1, S, Hq, D), 1), _rand((1, S, Hkv, D), 2), _rand((1, S, Hkv, D), 3), _rand((1, S, Hq, D), 4)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, m, scale)
    eps = 1e-6
    rng = np.random.default_rng(0)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(25):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            xp, xm = x.clone(), x.clone()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            fp = _loss(*[xp if a == name else args[a] for a in "qkv"], do, m, scale)
            fm = _loss(*[xm if a == name else args[a] for a in "qkv"], do, m, scale)
            num = (fp - fm) / (2 * eps)
            assert abs(num - float(g[idx])) <= 1e-7 * max(1.0, abs(num)), (name, idx, num, float(g[idx]))


def test_sdpa_autograd_special_case():
    S, H, D, scale = 19, 3, 16, 0.3
    m = _mask(1, S, [(0, 0, 0, (S,))])
    q, k, v, do = (_rand((1, S, H, D), 40 + i) for i in range(4))
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, m, scale)
    qq, kk, vv = (x.clone().transpose(1, 2).requires_grad_(True) for x in (q, k, v))
    out = F.scaled_dot_product_attention(qq, kk, vv, is_causal=True, scale=scale)
    out.backward(do.transpose(1, 2))
    for a, b in ((dq, qq.grad), (dk, kk.grad), (dv, vv.grad)):
        assert torch.allclose(a, b.transpose(1, 2), rtol=1e-10, atol=1e-12)


def test_gqa_matches_repeated_kv_heads():
    pl = [(0, 0, 5, (4, 3))]
    S, Hq, Hkv, D = 12, 4, 2, 8
    m = _mask(1, S, pl)
    q, k, v, do = _rand((1, S, Hq, D), 50), _rand((1, S, Hkv, D), 51), _rand((1, S, Hkv, D), 52), _rand((1, S, Hq, D), 53)
    kr, vr = k.repeat_interleave(2, dim=2), v.repeat_interleave(2, dim=2)
    O1, L1 = oracle.attn_fwd(q, k, v, m, 0.3)
    O2, L2 = oracle.attn_fwd(q, kr, vr, m, 0.3)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    _, dk1, dv1 = oracle.attn_bwd(q, k, v, do, m, 0.3)
    _, dk2, dv2 = oracle.attn_bwd(q, kr, vr, do, m, 0.3)
    assert torch.allclose(dk1, dk2.view(1, S, Hkv, 2, D).sum(3), atol=1e-12)
    assert torch.allclose(dv1, dv2.view(1, S, Hkv, 2, D).sum(3), atol=1e-12)


def test_negative_control_missing_jacobian_term_fails_fd():
    """Dropping the rowsum term of the softmax Jacobian must break the
    finite-difference agreement (so the check above can fail)."""
    pl = [(0, 0, 3, (2, 2))]
    S, H, D, scale = 7, 1, 4, 0.5
    m = torch.from_numpy(_mask(1, S, pl)[0])
    q, k, v, do = (_rand((1, S, H, D), 60 + i) for i in range(4))
    s = (q[0, :, 0] @ k[0, :, 0].T * scale).masked_fill(~m, float("-inf"))
    P = torch.softmax(s, dim=1)
    dP = do[0, :, 0] @ v[0, :, 0].T
    wrong_dq = (P * dP) @ k[0, :, 0] * scale
    dq, _, _ = oracle.attn_bwd(q, k, v, do, m[None].numpy(), scale)
    assert not torch.allclose(wrong_dq, dq[0, :, 0], atol=1e-6)


def test_sampled_equals_full():
    w = make_workload(None, 0, packset=PackSet(2, 40, [Pack(0, 0, 10, (12, 9)), Pack(1, 3, 0, (30,))]), heads=(4, 2, 16))
    P, R = descriptors([(p.row, p.start, p.prompt_len, p.resp_lens) for p in w.packset.packs])
    pk, br, _ = oracle.token_ids(P, R, 2, 40)
    m = oracle.attention_mask(pk, br)
    O, L = oracle.attn_fwd(w.q, w.k, w.v, m, w.scale)
    dq, dk, dv = oracle.attn_bwd(w.q, w.k, w.v, w.do, m, w.scale)
    rows = [0, 11, 25, 39]
    Os, Ls = oracle.attn_fwd_rows(w.q, w.k, w.v, m[1], 1, 3, rows, w.scale)
    assert torch.equal(Os, O[1, rows, 3]) and torch.equal(Ls, L[1, 3, rows])
    dqs, dks, dvs = oracle.attn_bwd_sampled(w.q, w.k, w.v, w.do, m[0], 0, 1, rows, [2, 30], w.scale)
    assert torch.allclose(dqs, torch.stack([dq[0, rows, 2], dq[0, rows, 3]]), atol=1e-14)
    assert torch.allclose(dks, dk[0, [2, 30], 1], atol=1e-14) and torch.allclose(dvs, dv[0, [2, 30], 1], atol=1e-14)


def test_mask_rows_match_the_full_mask():
    rng = np.random.default_rng(8)
    for _ in range(10):
        pl = [(0, 0, int(rng.integers(0, 6)), tuple(int(x) for x in rng.integers(0, 5, size=int(rng.integers(0, 4))))),
              (0, 20, int(rng.integers(0, 4)), (int(rng.integers(1, 4)),))]
        P, R = descriptors(pl)
        pk, br, _ = oracle.token_ids(P, R, 1, 30)
        full = oracle.attention_mask(pk, br, row=0)
        rows = rng.choice(30, size=7, replace=False)
        assert np.array_equal(oracle.attention_mask_rows(pk, br, 0, rows), full[rows])


def test_dq_rows_by_finite_differences():
    """attn_dq_rows is the gradient of <dO, O> with respect to the listed
    query rows (central differences on those rows), and it equals the full
    backward's rows."""
    pl = [(0, 0, 4, (3, 5)), (0, 12, 2, (2,)), (0, 17, 0, (3,))]
    S, Hq, Hkv, D, scale = 22, 4, 2, 8, 0.37
    m = _mask(1, S, pl)
    q, k, v, do = _rand((1, S, Hq, D), 61), _rand((1, S, Hkv, D), 62), _rand((1, S, Hkv, D), 63), _rand((1, S, Hq, D), 64)
    rows = [0, 3, 7, 8, 13, 16, 19, 21]
    h = 3
    dq_rows = oracle.attn_dq_rows(q, k, v, do, m[0][rows], 0, h, rows, scale)
    dq, _, _ = oracle.attn_bwd(q, k, v, do, m, scale)
    assert torch.allclose(dq_rows, dq[0, rows, h], atol=1e-13, rtol=0)
    eps = 1e-6
    for n, i in enumerate(rows):
        for d in (0, 5):
            qp, qm = q.clone(), q.clone()
            qp[0, i, h, d] += eps
            qm[0, i, h, d] -= eps
            num = (_loss(qp, k, v, do, m, scale) - _loss(qm, k, v, do, m, scale)) / (2 * eps)
            assert abs(num - float(dq_rows[n, d])) <= 1e-7 * max(1.0, abs(num))


def test_dkdv_rows_by_finite_differences():
    """attn_dkdv_rows is the gradient of <dO, O> with respect to the listed
    key rows (central differences on K and V, which every q head of the
    group shares), it equals the full backward's rows, and the query rows
    that see the listed keys are all it needs: at keys in the last tokens of
    a branch, the rows from the first listed key to the branch's end give
    the same values."""
    pl = [(0, 0, 4, (3, 5)), (0, 12, 2, (2,)), (0, 17, 0, (3,))]
    S, Hq, Hkv, D, scale = 22, 4, 2, 8, 0.37
    m = _mask(1, S, pl)
    q, k, v, do = _rand((1, S, Hq, D), 71), _rand((1, S, Hkv, D), 72), _rand((1, S, Hkv, D), 73), _rand((1, S, Hq, D), 74)
    _, dk, dv = oracle.attn_bwd(q, k, v, do, m, scale)
    every = list(range(S))
    keys = [0, 3, 4, 6, 9, 11, 12, 15, 18, 21]
    g = 1
    dk_rows, dv_rows = oracle.attn_dkdv_rows(q, k, v, do, m[0], 0, g, every, keys, scale)
    assert torch.allclose(dk_rows, dk[0, keys, g], atol=1e-13, rtol=0)
    assert torch.allclose(dv_rows, dv[0, keys, g], atol=1e-13, rtol=0)
    # the second response of the first pack is tokens 7..11: keys 9..11 are
    # seen by queries 9..11 only
    tail, qs = [9, 10, 11], [9, 10, 11]
    dk_t, dv_t = oracle.attn_dkdv_rows(q, k, v, do, m[0][qs], 0, g, qs, tail, scale)
    assert torch.allclose(dk_t, dk[0, tail, g], atol=1e-13, rtol=0)
    assert torch.allclose(dv_t, dv[0, tail, g], atol=1e-13, rtol=0)
    eps = 1e-6
    for n, j in enumerate(keys):
        for d in (0, 5):
            for x, got in ((k, dk_rows), (v, dv_rows)):
                xp, xm = x.clone(), x.clone()
                xp[0, j, g, d] += eps
                xm[0, j, g, d] -= eps
                args_p = (q, xp, v) if x is k else (q, k, xp)
                args_m = (q, xm, v) if x is k else (q, k, xm)
                num = (_loss(*args_p, do, m, scale) - _loss(*args_m, do, m, scale)) / (2 * eps)
                assert abs(num - float(got[n, d])) <= 1e-7 * max(1.0, abs(num))
