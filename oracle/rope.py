"""Rotary position embedding at branch-aligned positions, in fp64.  Test
infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use it.

"DPO Preference Packing: Dense Masks and Sparse Execution", section "Layout
requirements" (aligned positions): in a packed row every response keeps the
position ids it would have in its own [prompt | response] sequence, so the
prompt runs 0..p-1 and each response p..p+r-1 (the ids of
oracle.positions).  Rotary embedding turns those ids into rotations of
query and key head vectors.

The pages fix the positions, not the rotary convention.  Reading taken: the
rotate-half pairing of the Qwen3 family (head dim i pairs with i + D/2, for
i < D/2), frequencies base^(-2i/D):

    y[i]       = x[i] cos(pos f_i) - x[i + D/2] sin(pos f_i)
    y[i + D/2] = x[i] sin(pos f_i) + x[i + D/2] cos(pos f_i)

The backward of y = R(pos) x is dx = R(pos)^T dy = R(-pos) dy (a rotation's
transpose is its inverse).  The interleaved pairing (2i, 2i+1) is the same
rotation with the head dims permuted; it is provided for the pins.
"""
from __future__ import annotations

import numpy as np
import torch


def rope_freqs(D, base=10000.0):
    """f_i = base^(-2i/D), i = 0 .. D/2-1, fp64."""
    return base ** (-torch.arange(0, D // 2, dtype=torch.float64) * 2.0 / D)


def rope(x, pos, base=10000.0, inverse=False, interleaved=False):
    """Rotate x [..., T, H, D] (any float type, computed in fp64) at integer
    positions pos [T] (or broadcastable to x's token axis); inverse applies
    R(-pos).  Returns fp64."""
    x = torch.as_tensor(x).double()
    D = x.shape[-1]
    ang = torch.as_tensor(np.asarray(pos), dtype=torch.float64)[:, None] * rope_freqs(D, base)[None, :]
    if inverse:
        ang = -ang
    c, s = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]  # [T, 1, D/2]
    if interleaved:
        x1, x2 = x[..., 0::2], x[..., 1::2]
    else:
        x1, x2 = x[..., : D // 2], x[..., D // 2:]
    y1 = x1 * c - x2 * s
    y2 = x1 * s + x2 * c
    out = torch.empty_like(x)
    if interleaved:
        out[..., 0::2], out[..., 1::2] = y1, y2
    else:
        out[..., : D // 2], out[..., D // 2:] = y1, y2
    return out


def packed_rope(x, pos, base=10000.0, inverse=False):
    """x [B, S, H, D] at the packed position ids pos [B, S] (pad tokens carry
    position 0: the identity)."""
    x = torch.as_tensor(x).double()
    return torch.stack([rope(x[b], pos[b], base, inverse) for b in range(x.shape[0])])
