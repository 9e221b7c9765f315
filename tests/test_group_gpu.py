"""GPU group preference coefficients vs the oracle (fp64).

The kernel works in fp64 from the same fp32 inputs and rounds its outputs
to fp32, so coefficients, NLL weights and losses agree with the oracle to
fp32 rounding: |got - want| <= 1e-7 + 1e-6 |want|.  The end-to-end case
(logits -> packed token log-probs -> coefficients) compares with the oracle
run on the same logits; there the fp32 log-prob sums err by up to n * 1e-4
(their own bound), which moves u by at most beta * 1e-4 and a coefficient by
less than that over |G| (|d c / d u| <= 1 / |G| for every form).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import groupdpo as gd
from gpu_path import api, say
from workloads.generate import descriptor_arrays, make_packset, random_packset

pytestmark = pytest.mark.gpu


def _random_batch(rng, n_resp, n_groups, kmax, share):
    """Groups over n_resp responses; with `share`, groups draw members from a
    common pool so that responses recur across groups."""
    groups = []
    nxt = 0
    for _ in range(n_groups):
        k = int(rng.integers(2, kmax + 1))
        if share:
            m = rng.choice(n_resp, size=k, replace=False).tolist()
        else:
            m = list(range(nxt, nxt + k))
            nxt += k
        npos = int(rng.integers(1, k))
        groups.append((m[:npos], m[npos:]))
    n_all = max(n_resp, nxt + 4)  # without sharing, a few responses in no group
    lens = rng.integers(1, 1500, size=n_all).astype(np.int32)
    pol = (-lens * rng.uniform(0.2, 3.0, size=n_all)).astype(np.float32)
    ref = (-lens * rng.uniform(0.2, 3.0, size=n_all)).astype(np.float32)
    return groups, lens, pol, ref


def _csr(groups):
    ptr, mem, pos = [0], [], []
    for P, N in groups:
        mem += list(P) + list(N)
        pos += [1] * len(P) + [0] * len(N)
        ptr.append(len(mem))
    return (torch.tensor(ptr, dtype=torch.int32), torch.tensor(mem, dtype=torch.int32),
            torch.tensor(pos, dtype=torch.uint8))


def _gpu(groups, lens, pol, ref, beta, obj, alpha=1.0):
    A = api()
    gp, mem, pos = (t.cuda() for t in _csr(groups))
    coef, nll_w, loss, st = A.group_coefficients(gp, mem, pos, torch.from_numpy(pol).cuda(),
                                                 torch.from_numpy(ref).cuda(), torch.from_numpy(lens).cuda(),
                                                 beta, obj, alpha)
    torch.cuda.synchronize()
    return (coef.cpu().double().numpy(), nll_w.cpu().double().numpy(), loss.cpu().double().numpy(),
            tuple(st.cpu().tolist()))


def _want(groups, lens, pol, ref, beta, obj, alpha=1.0):
    u = gd.implicit_rewards(pol.astype(np.float64), ref.astype(np.float64), lens, beta)
    p = pol.astype(np.float64) / lens
    return (gd.group_coefficients(obj, groups, u), gd.positive_nll_weights(groups, len(lens), alpha),
            np.array([gd.group_objective(obj, groups, u), gd.positive_nll(groups, p, alpha)]))


def _close(got, want, what):
    err = np.abs(got - want)
    assert (err <= 1e-7 + 1e-6 * np.abs(want)).all(), (what, float(err.max()))


@pytest.mark.parametrize("obj", gd.OBJECTIVES)
@pytest.mark.parametrize("seed", range(3))
def test_random_groups(obj, seed):
    rng = np.random.default_rng(500 + seed)
    share = seed == 2
    n_groups = [3, 40, 25][seed]
    n_resp = [12, 300, 30][seed]
    groups, lens, pol, ref = _random_batch(rng, n_resp, n_groups, kmax=[3, 7, 6][seed], share=share)
    n_resp = len(lens)
    beta = [0.1, 0.05, 2.0][seed]
    say("group", obj, seed, len(groups), n_resp)
    coef, nll_w, loss, st = _gpu(groups, lens, pol, ref, beta, obj, alpha=[1.0, 0.5, 0.0][seed])
    assert st == (0, 0)
    c, w, l = _want(groups, lens, pol, ref, beta, obj, alpha=[1.0, 0.5, 0.0][seed])
    _close(coef, c, "coef")
    _close(nll_w, w, "nll_w")
    _close(loss, l, "loss")


@pytest.mark.parametrize("obj", gd.OBJECTIVES)
def test_extreme_rewards_and_largest_batch(obj):
    rng = np.random.default_rng(7)
    # 2048 groups of 2 = the maximum entry count; huge reward gaps
    n = 4096
    groups = [([2 * g], [2 * g + 1]) for g in range(n // 2)]
    lens = np.ones(n, dtype=np.int32)
    pol = rng.choice([-2000.0, -1.0, -0.5], size=n).astype(np.float32)
    ref = rng.choice([-2000.0, -1.0, -0.5], size=n).astype(np.float32)
    say("group extreme", obj)
    coef, nll_w, loss, st = _gpu(groups, lens, pol, ref, 1.0, obj)
    assert st == (0, 0) and np.isfinite(coef).all() and np.isfinite(loss).all()
    c, w, l = _want(groups, lens, pol, ref, 1.0, obj)
    _close(coef, c, "coef")
    _close(nll_w, w, "nll_w")
    _close(loss, l, "loss")


def test_deterministic():
    rng = np.random.default_rng(11)
    groups, lens, pol, ref = _random_batch(rng, 64, 50, 6, share=True)
    a = _gpu(groups, lens, pol, ref, 0.1, "softmax")
    b = _gpu(groups, lens, pol, ref, 0.1, "softmax")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[2], b[2])


def test_bad_groups_set_status_and_nan():
    lens = np.full(6, 10, dtype=np.int32)
    pol = np.full(6, -5.0, dtype=np.float32)
    ref = pol.copy()
    cases = {
        15: [([0], [1]), ([2, 3], [])],          # no negative in group 1
        14: [([0], [1]), ([2], [3]), ([4], [4])],  # response 4 both positive and negative
        12: [([0], [1]), ([7], [2])],             # member outside [0, 6)
    }
    for code, groups in cases.items():
        say("group status", code)
        coef, nll_w, loss, st = _gpu(groups, lens, pol, ref, 0.1, "all_pairs")
        bad = next(i for i, (P, N) in enumerate(groups) if gd.validate_groups([(P, N)], 6) == 0)
        assert st == (code, bad)
        assert np.isnan(coef).all() and np.isnan(nll_w).all() and np.isnan(loss).all()
    bad_len = lens.copy()
    bad_len[3] = 0
    _, _, _, st = _gpu([([0], [1]), ([2], [3])], bad_len, pol, ref, 0.1, "mpo")
    assert st == (13, 1)
    # group_ptr that does not end at n_entries
    A = api()
    gp = torch.tensor([0, 2, 3], dtype=torch.int32).cuda()
    mem = torch.tensor([0, 1, 2, 3], dtype=torch.int32).cuda()
    pos = torch.tensor([1, 0, 1, 0], dtype=torch.uint8).cuda()
    t = lambda x: torch.from_numpy(x).cuda()  # noqa: E731
    _, _, _, st = A.group_coefficients(gp, mem, pos, t(pol), t(ref), t(lens), 0.1)
    assert tuple(st.cpu().tolist()) == (11, 1)


@pytest.mark.parametrize("cfg", [1, 2, 5])
def test_from_packed_logprobs(cfg):
    """logits -> packed token log-probs (policy and reference) -> group
    coefficients, each pack one group with response 0 preferred (config 5:
    its first four responses preferred)."""
    ps = make_packset(cfg)
    A = api()
    V = 512
    g = torch.Generator().manual_seed(40 + cfg)
    lp = (torch.randn((ps.B, ps.S, V), generator=g) * 2.0).to(torch.bfloat16)
    lr = (torch.randn((ps.B, ps.S, V), generator=g) * 2.0).to(torch.bfloat16)
    tokens = torch.randint(0, V, (ps.B, ps.S), generator=g, dtype=torch.int32)
    P, R = descriptor_arrays(ps)
    pd, rd = A.descriptors_to_device(P, R)
    m = A.pack_block_map(pd, rd, ps.B, ps.S, 64, 64)
    _, src, mask = A.pack_positions(m)
    _, pol = A.packed_token_logp(m, src, mask, lp.cuda().contiguous(), tokens.cuda(), pd, rd)
    _, ref = A.packed_token_logp(m, src, mask, lr.cuda().contiguous(), tokens.cuda(), pd, rd)
    nresp = [int(x) for x in np.asarray(P).reshape(-1, 5)[:, 3]]
    flags = []
    for k in nresp:
        flags += [1] * (k // 2 if k > 2 else 1) + [0] * (k - (k // 2 if k > 2 else 1))
    gp, mem, pos = A.groups_from_packs(nresp, flags)
    lens = torch.as_tensor(np.asarray(R, dtype=np.int32))
    beta = 0.1
    say("group from packs", cfg, len(nresp))
    # the oracle from the same logits
    _, osrc, omask, _ = oracle.positions(P, R, ps.B, ps.S)
    lpf, lrf = lp.float(), lr.float()
    tp = oracle.token_logp(lambda b, r: lpf[b, r].numpy(), tokens.numpy(), osrc, omask)
    tr = oracle.token_logp(lambda b, r: lrf[b, r].numpy(), tokens.numpy(), osrc, omask)
    rp, rr = oracle.response_logp(P, R, tp), oracle.response_logp(P, R, tr)
    groups, e = [], 0
    for k in nresp:
        fl = flags[e:e + k]
        groups.append(([e + i for i in range(k) if fl[i]], [e + i for i in range(k) if not fl[i]]))
        e += k
    L = np.asarray(R, dtype=np.float64)
    u = gd.implicit_rewards(rp, rr, L, beta)
    for obj in gd.OBJECTIVES:
        coef, nll_w, loss, st = A.group_coefficients(gp.cuda(), mem.cuda(), pos.cuda(), pol, ref, lens.cuda(), beta,
                                                     obj)
        torch.cuda.synchronize()
        assert tuple(st.cpu().tolist()) == (0, 0)
        c = gd.group_coefficients(obj, groups, u)
        # |du| <= 2 beta 1e-4 per response; the Hessian rows of every form sum
        # to at most 1 in absolute value, and c carries 1/|G|
        assert np.abs(coef.cpu().double().numpy() - c).max() <= beta * 2e-4 / len(groups) + 1e-6
        want_loss = gd.group_objective(obj, groups, u)
        assert abs(float(loss[0]) - want_loss) <= beta * 4e-4 + 1e-6
        _close(nll_w.cpu().double().numpy(), gd.positive_nll_weights(groups, len(L)), "nll_w")
