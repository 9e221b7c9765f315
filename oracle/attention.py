"""Dense fp64 masked attention and its naive backward (CPU, torch float64).

This is ordinary softmax attention with an explicit boolean mask (the dense
form p1 "Dense and sparse execution" writes as scores = q k^T followed by a
masked fill), evaluated in float64 from the bf16 inputs (exact conversion).

Readings where the pages are silent:
  * softmax scale is an argument (the workloads use 1/sqrt(head_dim));
  * grouped heads: q head h reads kv head floor(h / (Hq / Hkv));
  * LSE is the natural log of the sum of exp(scaled scores); a query with
    no allowed key (pad) gets O = 0 and LSE = -inf, and its gradients and
    those of pad keys are 0;
  * the backward differentiates the softmax directly:
    dS = P * (dP - rowsum(P * dP)), with dP = dO V^T.
"""
from __future__ import annotations

import math

import numpy as np
import torch

_F64 = torch.float64


def _t(x):
    if isinstance(x, np.ndarray):
        x = torch.from_numpy(x)
    return x.to(_F64)


def _probs(qh, kg, m, scale):
    """Row softmax of scale * qh kg^T under mask m; rows with no key -> 0."""
    s = (qh @ kg.T) * scale
    s = s.masked_fill(~m, float("-inf"))
    valid = m.any(dim=1)
    mx = torch.where(valid, s.max(dim=1).values, torch.zeros((), dtype=_F64))
    e = torch.exp(s - mx[:, None])          # exp(-inf) = 0 on masked entries
    l = e.sum(dim=1)
    P = torch.where(valid[:, None], e / torch.where(valid, l, torch.ones((), dtype=_F64))[:, None],
                    torch.zeros((), dtype=_F64))
    lse = torch.where(valid, mx + torch.log(torch.where(valid, l, torch.ones((), dtype=_F64))),
                      torch.full((), float("-inf"), dtype=_F64))
    return P, lse


def attn_fwd(q, k, v, mask, scale, rows=None, heads=None):
    """O [B, S, Hq, D] and LSE [B, Hq, S] in float64.

    q: [B, S, Hq, D], k, v: [B, S, Hkv, D] (any float dtype), mask: bool
    [B, S, S].  `rows` / `heads` restrict the work to some batch rows and
    q heads (other entries stay 0 / -inf).
    """
    q, k, v = _t(q), _t(k), _t(v)
    B, S, Hq, D = q.shape
    G = Hq // k.shape[2]
    O = torch.zeros((B, S, Hq, D), dtype=_F64)
    LSE = torch.full((B, Hq, S), float("-inf"), dtype=_F64)
    for b in (range(B) if rows is None else rows):
        m = torch.from_numpy(np.ascontiguousarray(mask[b]))
        for h in (range(Hq) if heads is None else heads):
            g = h // G
            P, lse = _probs(q[b, :, h], k[b, :, g], m, scale)
            O[b, :, h] = P @ v[b, :, g]
            LSE[b, h] = lse
    return O, LSE


def attn_bwd(q, k, v, do, mask, scale, rows=None, groups=None):
    """dQ [B, S, Hq, D], dK, dV [B, S, Hkv, D] in float64 for the loss
    <dO, O>.  dK / dV sum the contributions of every q head in the group.
    `rows` / `groups` restrict the work to some batch rows and kv heads."""
    q, k, v, do = _t(q), _t(k), _t(v), _t(do)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    dq = torch.zeros_like(q)
    dk = torch.zeros_like(k)
    dv = torch.zeros_like(v)
    for b in (range(B) if rows is None else rows):
        m = torch.from_numpy(np.ascontiguousarray(mask[b]))
        for g in (range(Hkv) if groups is None else groups):
            for h in range(g * G, (g + 1) * G):
                P, _ = _probs(q[b, :, h], k[b, :, g], m, scale)
                dP = do[b, :, h] @ v[b, :, g].T
                dS = P * (dP - (P * dP).sum(dim=1, keepdim=True))
                dq[b, :, h] = (dS @ k[b, :, g]) * scale
                dk[b, :, g] += (dS.T @ q[b, :, h]) * scale
                dv[b, :, g] += P.T @ do[b, :, h]
    return dq, dk, dv


def attn_fwd_rows(q, k, v, mask_b, b, h, qrows, scale):
    """O [n, D] and LSE [n] of the listed query rows of (batch row b, q head h)."""
    q, k, v = _t(q), _t(k), _t(v)
    G = q.shape[2] // k.shape[2]
    g = h // G
    idx = torch.as_tensor(np.asarray(qrows), dtype=torch.long)
    m = torch.from_numpy(np.ascontiguousarray(mask_b[np.asarray(qrows)]))
    P, lse = _probs(q[b, idx, h], k[b, :, g], m, scale)
    return P @ v[b, :, g], lse


def attn_dq_rows(q, k, v, do, mask_rows, b, h, qrows, scale):
    """dQ [n, D] of the listed query rows of (batch row b, q head h) for the
    loss <dO, O>, each row from its own softmax: P_i, O_i = P_i V, the row dot
    product Delta_i = dO_i . O_i, dS_ij = P_ij (dO_i . V_j - Delta_i) and
    dQ_i = scale sum_j dS_ij K_j.  mask_rows [n, S] are those rows of the
    mask (so that very long rows need no S x S mask)."""
    q, k, v, do = _t(q), _t(k), _t(v), _t(do)
    G = q.shape[2] // k.shape[2]
    g = h // G
    idx = torch.as_tensor(np.asarray(qrows), dtype=torch.long)
    m = torch.from_numpy(np.ascontiguousarray(mask_rows))
    P, _ = _probs(q[b, idx, h], k[b, :, g], m, scale)
    O = P @ v[b, :, g]
    dOi = do[b, idx, h]
    delta = (dOi * O).sum(dim=1)
    dS = P * (dOi @ v[b, :, g].T - delta[:, None])
    return scale * (dS @ k[b, :, g])


def attn_dkdv_rows(q, k, v, do, mask_rows, b, g, qrows, krows, scale):
    """dK [m, D] and dV [m, D] of the listed key rows of (batch row b, kv
    group g) for the loss <dO, O>, summed over the group's q heads.
    mask_rows [n, S] are the mask rows of the query rows qrows, which must
    hold every query that sees a listed key (no other query contributes to
    those keys).  Each query's softmax comes from its own full row: P_i,
    O_i = P_i V, Delta_i = dO_i . O_i; for a listed key j,
    dS_ij = P_ij (dO_i . V_j - Delta_i), dV_j = sum_i P_ij dO_i and
    dK_j = scale sum_i dS_ij Q_i (so that very long rows need no S x S
    mask)."""
    q, k, v, do = _t(q), _t(k), _t(v), _t(do)
    G = q.shape[2] // k.shape[2]
    qi = torch.as_tensor(np.asarray(qrows), dtype=torch.long)
    kj = torch.as_tensor(np.asarray(krows), dtype=torch.long)
    m = torch.from_numpy(np.ascontiguousarray(mask_rows))
    kg, vg = k[b, :, g], v[b, :, g]
    dk = torch.zeros((len(kj), k.shape[3]), dtype=torch.float64)
    dv = torch.zeros_like(dk)
    for h in range(g * G, (g + 1) * G):
        P, _ = _probs(q[b, qi, h], kg, m, scale)
        dOi = do[b, qi, h]
        delta = (dOi * (P @ vg)).sum(dim=1)
        Pj = P[:, kj]
        dS = Pj * (dOi @ vg[kj].T - delta[:, None])
        dv += Pj.T @ dOi
        dk += scale * (dS.T @ q[b, qi, h])
    return dk, dv


def attn_bwd_sampled(q, k, v, do, mask_b, b, g, qrows, krows, scale):
    """Gradients at sampled positions of batch row b and kv group g:
    dQ[qrows] for every q head of the group ([G, n, D]) and dK[krows],
    dV[krows] ([n, D]).  Computes the group's full backward for that row."""
    B = q.shape[0]
    sub = lambda x: x[b:b + 1]  # noqa: E731
    dq, dk, dv = attn_bwd(sub(q), sub(k), sub(v), sub(do), mask_b[None], scale, groups=[g])
    G = q.shape[2] // k.shape[2]
    qi = torch.as_tensor(np.asarray(qrows), dtype=torch.long)
    ki = torch.as_tensor(np.asarray(krows), dtype=torch.long)
    dq_s = torch.stack([dq[0, qi, h] for h in range(g * G, (g + 1) * G)])
    return dq_s, dk[0, ki, g], dv[0, ki, g]


def useful_flops(n_allowed: int, Hq: int, D: int) -> float:
    """fwd+bwd FLOPs counting only allowed (query, key) pairs: 4*D per pair
    forward (Q K^T and P V), 10*D backward (Q K^T recompute, dO V^T, P^T dO,
    dS K, dS^T Q), per q head."""
    return 14.0 * D * Hq * float(n_allowed)
