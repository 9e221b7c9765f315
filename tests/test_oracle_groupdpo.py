"""Pins of the oracle's group preference objectives and surrogate
coefficients (CPU only).

What fixes them: for one positive and one negative every objective is the
DPO loss -log sigmoid(u_+ - u_-) (a closed form); hand-evaluated values at
u = 0 tell the four forms apart; the coefficients equal central finite
differences of L_group; each group's gradient sums to zero (every form
depends on differences of u only); a response shared by two groups gets
the sum of both groups' terms; the NLL weights have a closed form; the
forms agree with one another where their definitions meet (one positive,
members with equal rewards) and none depends on the order of members.
"""
import math

import numpy as np
import pytest

from oracle import groupdpo as gd


def _dpo(d):
    return math.log1p(math.exp(-d))  # -log sigmoid(d), d moderate


@pytest.mark.parametrize("obj", gd.OBJECTIVES)
@pytest.mark.parametrize("up,un", [(0.0, 0.0), (1.5, -0.25), (-3.0, 2.0), (0.125, 0.125)])
def test_one_pair_is_the_dpo_loss(obj, up, un):
    assert abs(gd.phi(obj, [up], [un]) - _dpo(up - un)) < 1e-14
    gP, gN = gd.phi_grad(obj, [up], [un])
    s = 1.0 / (1.0 + math.exp(up - un))  # sigmoid(u_- - u_+)
    assert abs(gP[0] + s) < 1e-14 and abs(gN[0] - s) < 1e-14


def test_hand_values_at_zero_tell_the_forms_apart():
    ln2, ln3 = math.log(2.0), math.log(3.0)
    # one positive, two negatives, all at u = 0
    want = {"all_pairs": ln2, "margin": ln2, "mpo": ln3, "softmax": ln3}
    for obj, v in want.items():
        assert abs(gd.phi(obj, [0.0], [0.0, 0.0]) - v) < 1e-14, obj
    # two positives, one negative
    want = {"all_pairs": ln2, "margin": ln2, "mpo": math.log(1.5), "softmax": ln2}
    for obj, v in want.items():
        assert abs(gd.phi(obj, [0.0, 0.0], [0.0]) - v) < 1e-14, obj
    # margin compares means: P = {2, 0}, N = {1}: -log sigmoid(0)
    assert abs(gd.phi("margin", [2.0, 0.0], [1.0]) - ln2) < 1e-14
    # all-pairs averages pair losses: P = {1}, N = {0, 2}
    assert abs(gd.phi("all_pairs", [1.0], [0.0, 2.0]) - 0.5 * (_dpo(1.0) + _dpo(-1.0))) < 1e-14


def _random_groups(rng, n_resp, n_groups, kmax=5):
    groups = []
    for _ in range(n_groups):
        k = int(rng.integers(2, kmax + 1))
        m = rng.choice(n_resp, size=k, replace=False).tolist()
        npos = int(rng.integers(1, k))
        groups.append((m[:npos], m[npos:]))
    return groups


@pytest.mark.parametrize("obj", gd.OBJECTIVES)
@pytest.mark.parametrize("seed", range(4))
def test_coefficients_match_finite_differences(obj, seed):
    rng = np.random.default_rng(seed)
    n = 12
    groups = _random_groups(rng, n, 6)
    u = rng.normal(0, 2, size=n)
    c = gd.group_coefficients(obj, groups, u)
    h = 1e-5
    for i in range(n):
        e = np.zeros(n)
        e[i] = h
        fd = (gd.group_objective(obj, groups, u + e) - gd.group_objective(obj, groups, u - e)) / (2 * h)
        assert abs(fd - c[i]) < 1e-8, (obj, i, fd, c[i])


@pytest.mark.parametrize("obj", gd.OBJECTIVES)
def test_group_gradient_sums_to_zero_and_shift_invariance(obj):
    rng = np.random.default_rng(9)
    for _ in range(20):
        k = int(rng.integers(2, 9))
        npos = int(rng.integers(1, k))
        u = rng.normal(0, 3, size=k)
        gP, gN = gd.phi_grad(obj, u[:npos], u[npos:])
        assert abs(gP.sum() + gN.sum()) < 1e-13
        v0 = gd.phi(obj, u[:npos], u[npos:])
        v1 = gd.phi(obj, u[:npos] + 7.0, u[npos:] + 7.0)
        assert abs(v0 - v1) < 1e-12


@pytest.mark.parametrize("obj", gd.OBJECTIVES)
def test_shared_response_accumulates(obj):
    rng = np.random.default_rng(4)
    u = rng.normal(0, 1, size=5)
    g1, g2 = ([0], [1, 2]), ([3, 1], [4])  # response 1: negative in g1, positive in g2
    c = gd.group_coefficients(obj, [g1, g2], u)
    a = gd.group_coefficients(obj, [g1], u)
    b = gd.group_coefficients(obj, [g2], u)
    assert np.allclose(c, (a + b) / 2, atol=1e-15, rtol=0)  # 1/|G| with |G| = 2
    assert c[1] == pytest.approx((a[1] + b[1]) / 2, abs=1e-15)


@pytest.mark.parametrize("obj", gd.OBJECTIVES)
def test_extreme_rewards_stay_finite(obj):
    for up, un in [([900.0, -900.0], [0.0]), ([-1e3], [1e3, -1e3]), ([1e3, 1e3], [1e3 - 1e-9])]:
        v = gd.phi(obj, up, un)
        gP, gN = gd.phi_grad(obj, up, un)
        assert np.isfinite(v) and np.all(np.isfinite(gP)) and np.all(np.isfinite(gN))
        assert abs(gP.sum() + gN.sum()) < 1e-12


def test_implicit_rewards_length_normalised():
    u = gd.implicit_rewards([-30.0, -12.0], [-20.0, -16.0], [10, 4], 0.1)
    assert np.allclose(u, [0.1 * (-3.0 + 2.0), 0.1 * (-3.0 + 4.0)], atol=1e-15, rtol=0)


def test_positive_nll_weights_closed_form():
    groups = [([0, 1], [2]), ([1], [3, 4]), ([5], [0])]
    w = gd.positive_nll_weights(groups, 6, alpha=1.0)
    want = np.array([1 / 6, 1 / 6 + 1 / 3, 0, 0, 0, 1 / 3])
    assert np.allclose(w, want, atol=1e-15, rtol=0)
    p = np.array([-1.0, -2.0, -3.0, -4.0, -5.0, -6.0])
    # the NLL value is linear in -p with exactly these weights
    assert abs(gd.positive_nll(groups, p) - float(w @ -p)) < 1e-14


def test_validation():
    assert gd.validate_groups([([0], [1]), ([2], [3])], 4) == -1
    assert gd.validate_groups([([0], [1]), ([], [3])], 4) == 1      # empty positives
    assert gd.validate_groups([([0], [])], 4) == 0                  # empty negatives
    assert gd.validate_groups([([0], [1]), ([2], [2])], 4) == 1     # positive and negative
    assert gd.validate_groups([([0, 0], [1])], 4) == 0              # duplicate
    assert gd.validate_groups([([0], [4])], 4) == 0                 # out of range


def test_forms_agree_where_their_definitions_meet():
    """Cross-checks between the forms (each computed by its own branch of
    the oracle): with one positive, MPO and the softmax form are both the
    negative log-probability of the positive under a softmax over the group;
    when all positives share one reward and all negatives another, all-pairs
    and margin reduce to the one-pair DPO loss and the softmax form to the
    one-positive case; none depends on the order of members; all tend to 0
    as the negatives' rewards fall."""
    rng = np.random.default_rng(17)
    for k in range(1, 6):
        up = float(rng.normal())
        un = rng.normal(size=k)
        z = np.concatenate([[up], un])
        want = float(np.log(np.exp(z - z.max()).sum()) + z.max() - up)
        assert abs(gd.phi("mpo", [up], un) - want) < 1e-13
        assert abs(gd.phi("softmax", [up], un) - want) < 1e-13
    for nP in (1, 2, 4):
        for nN in (1, 3):
            a, b = float(rng.normal()), float(rng.normal())
            for obj in ("all_pairs", "margin"):
                assert abs(gd.phi(obj, [a] * nP, [b] * nN) - _dpo(a - b)) < 1e-13, obj
            one = gd.phi("softmax", [a], [b] * nN)
            assert abs(gd.phi("softmax", [a] * nP, [b] * nN) - one) < 1e-13
    for obj in gd.OBJECTIVES:
        uP, uN = rng.normal(size=3), rng.normal(size=4)
        base = gd.phi(obj, uP, uN)
        assert abs(gd.phi(obj, uP[::-1], rng.permutation(uN)) - base) < 1e-13, obj
        assert 0.0 <= gd.phi(obj, uP, uN - 60.0) < 1e-20, obj
