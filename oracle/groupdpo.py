"""Group preference objectives and their first-order surrogate
coefficients, in fp64.  Test infrastructure: only the tests, the smoke check
and the benchmark's CPU baseline use it.

"GroupDPO" page, section "core formulas": a batch holds a set G of groups;
group g has non-empty, disjoint sets of positive responses P_g and negative
responses N_g (a response may belong to several groups).  With p_i and r_i
the length-normalised (mean per token) log-probs of response i under the
policy and the frozen reference,

    u_i     = beta (p_i - r_i)
    L_group = (1/|G|) sum_g phi_g(u[P_g], u[N_g])
    c_i     = (1/|G|) sum_{g containing i} d phi_g / d u_i   (at the current u)

and L_sur = sum_i stopgrad(c_i) u_i has the same first-order gradient as
L_group.  The default adds a positive-response NLL term: the mean over a
group's positives of their mean token NLL (-p_i), then the mean over the
batch's groups, times alpha (alpha = 1).

The page names four group objectives (Margin, MPO, Softmax, All-Pairs) but
does not write them out; the forms below are the plainest readings, each
reducing to the DPO loss -log sigmoid(u_+ - u_-) for one positive and one
negative:

    all_pairs  mean over (i in P, j in N) of -log sigmoid(u_i - u_j)
    margin     -log sigmoid(mean_P u - mean_N u)
    mpo        -log( sum_P e^u / sum_{P u N} e^u )   (log-sum-exp form, as
               the page asks, so that a small positive mass does not divide)
    softmax    mean over i in P of -log( e^{u_i} / (e^{u_i} + sum_N e^u) )

Gradients are written out analytically from these definitions; the tests
pin them against central finite differences of the values.
"""
from __future__ import annotations

import math

import numpy as np

OBJECTIVES = ("all_pairs", "margin", "mpo", "softmax")


def log_sigmoid(x):
    """log(1 / (1 + e^-x)), stable for large |x|."""
    x = float(x)
    return -math.log1p(math.exp(-x)) if x >= 0 else x - math.log1p(math.exp(x))


def sigmoid(x):
    x = float(x)
    if x >= 0:
        return 1.0 / (1.0 + math.exp(-x))
    e = math.exp(x)
    return e / (1.0 + e)


def logsumexp(v):
    v = np.asarray(v, dtype=np.float64)
    m = v.max()
    return float(m + np.log(np.exp(v - m).sum()))


def implicit_rewards(policy_sum, ref_sum, resp_len, beta):
    """u_i = beta (p_i - r_i) from per-response log-prob SUMS (the packed
    log-prob kernel's output) and response lengths: p_i = sum_i / len_i."""
    L = np.asarray(resp_len, dtype=np.float64)
    return beta * (np.asarray(policy_sum, np.float64) / L - np.asarray(ref_sum, np.float64) / L)


def phi(objective, uP, uN):
    """Value of one group's objective."""
    uP = np.asarray(uP, dtype=np.float64)
    uN = np.asarray(uN, dtype=np.float64)
    if objective == "all_pairs":
        return float(np.mean([-log_sigmoid(a - b) for a in uP for b in uN]))
    if objective == "margin":
        return -log_sigmoid(uP.mean() - uN.mean())
    if objective == "mpo":
        return logsumexp(np.concatenate([uP, uN])) - logsumexp(uP)
    if objective == "softmax":
        return float(np.mean([logsumexp(np.concatenate([[a], uN])) - a for a in uP]))
    raise ValueError(objective)


def phi_grad(objective, uP, uN):
    """(d phi / d uP, d phi / d uN) of one group, analytically."""
    uP = np.asarray(uP, dtype=np.float64)
    uN = np.asarray(uN, dtype=np.float64)
    nP, nN = len(uP), len(uN)
    gP = np.zeros(nP)
    gN = np.zeros(nN)
    if objective == "all_pairs":
        # d/dx of -log sigmoid(x) is -sigmoid(-x), x = u_i - u_j
        for i in range(nP):
            for j in range(nN):
                s = sigmoid(uN[j] - uP[i]) / (nP * nN)
                gP[i] -= s
                gN[j] += s
    elif objective == "margin":
        s = sigmoid(uN.mean() - uP.mean())
        gP[:] = -s / nP
        gN[:] = s / nN
    elif objective == "mpo":
        allu = np.concatenate([uP, uN])
        w_all = np.exp(allu - allu.max())
        w_all /= w_all.sum()
        w_pos = np.exp(uP - uP.max())
        w_pos /= w_pos.sum()
        gP[:] = w_all[:nP] - w_pos
        gN[:] = w_all[nP:]
    elif objective == "softmax":
        for i in range(nP):
            z = np.concatenate([[uP[i]], uN])
            w = np.exp(z - z.max())
            w /= w.sum()
            gP[i] += (w[0] - 1.0) / nP
            gN += w[1:] / nP
    else:
        raise ValueError(objective)
    return gP, gN


def validate_groups(groups, n_resp):
    """Index of the first invalid group, else -1.  A group is (P, N) with
    non-empty P and N, members in [0, n_resp) and no response twice within
    the group (which also rules out a response both positive and negative)."""
    for gi, (P, N) in enumerate(groups):
        m = list(P) + list(N)
        if not P or not N or len(set(m)) != len(m) or any(i < 0 or i >= n_resp for i in m):
            return gi
    return -1


def group_objective(objective, groups, u):
    """L_group = (1/|G|) sum_g phi_g."""
    u = np.asarray(u, dtype=np.float64)
    return sum(phi(objective, u[list(P)], u[list(N)]) for P, N in groups) / len(groups)


def group_coefficients(objective, groups, u):
    """c_i = (1/|G|) sum_{g containing i} d phi_g / d u_i; responses in no
    group get 0."""
    u = np.asarray(u, dtype=np.float64)
    c = np.zeros(len(u))
    for P, N in groups:
        gP, gN = phi_grad(objective, u[list(P)], u[list(N)])
        for i, x in zip(P, gP):
            c[i] += x
        for j, x in zip(N, gN):
            c[j] += x
    return c / len(groups)


def positive_nll_weights(groups, n_resp, alpha=1.0):
    """Weight of each response's mean token NLL (-p_i) in the NLL term:
    alpha * sum_{g: i in P_g} 1 / (|G| |P_g|)."""
    w = np.zeros(n_resp)
    for P, _ in groups:
        for i in P:
            w[i] += alpha / (len(groups) * len(P))
    return w


def positive_nll(groups, p, alpha=1.0):
    """alpha * (1/|G|) sum_g mean_{i in P_g} (-p_i)."""
    p = np.asarray(p, dtype=np.float64)
    return alpha * sum(float(np.mean(-p[list(P)])) for P, _ in groups) / len(groups)
