"""Independent constructions the oracle is pinned against (test helpers).

Nothing here is used by the oracle itself.  The mask is rebuilt as a union
of ordinary causal sequences: pack p with responses r_1..r_K is the set of
pairwise sequences [prompt | r_k] (p1 "Layout requirements"; just [prompt]
for a pack without responses), and a (query, key) pair is allowed when some
such sequence holds both tokens with the key at or before the query.
"""
from __future__ import annotations

import itertools

import numpy as np


def pairwise_union_mask(B, S, packs_list):
    """packs_list: iterable of (row, start, prompt_len, resp_lens)."""
    m = np.zeros((B, S, S), dtype=bool)
    for row, start, plen, rls in packs_list:
        prompt = list(range(start, start + plen))
        seqs = []
        pos = start + plen
        for r in rls:
            seqs.append(prompt + list(range(pos, pos + r)))
            pos += r
        if not rls:
            seqs.append(prompt)
        for seq in seqs:
            for a, qi in enumerate(seq):
                for kj in seq[:a + 1]:
                    m[row, qi, kj] = True
    return m


def closed_form_count(packs_list):
    """Allowed pairs of a pack set: each pack contributes the causal prompt
    triangle p(p+1)/2 plus, per response k, r_k*p (all of the prompt) and its
    own causal triangle r_k(r_k+1)/2."""
    tot = 0
    for _, _, p, rls in packs_list:
        tot += p * (p + 1) // 2
        for r in rls:
            tot += r * p + r * (r + 1) // 2
    return tot


def descriptors(packs_list):
    rows, lens = [], []
    for row, start, plen, rls in packs_list:
        rows.append((row, start, plen, len(rls), len(lens)))
        lens.extend(rls)
    return np.asarray(rows, dtype=np.int32).reshape(-1, 5), np.asarray(lens, dtype=np.int32)


def small_single_packs():
    """Every single pack with prompt 0-4 and 0-3 responses of 0-3 tokens (425)."""
    for p in range(5):
        for k in range(4):
            for rls in itertools.product(range(4), repeat=k):
                yield p, tuple(rls)


def rope(x, pos, base=10000.0):
    """Rotary position encoding of x [T, H, D] (fp64) at integer positions pos [T]
    (pairs (2i, 2i+1) rotated by pos * base^(-2i/D)); test-only helper."""
    import torch
    T, H, D = x.shape
    inv = base ** (-torch.arange(0, D, 2, dtype=torch.float64) / D)
    ang = torch.as_tensor(pos, dtype=torch.float64)[:, None] * inv[None, :]
    c, s = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]
    x1, x2 = x[..., 0::2], x[..., 1::2]
    out = torch.empty_like(x)
    out[..., 0::2] = x1 * c - x2 * s
    out[..., 1::2] = x1 * s + x2 * c
    return out
