"""Runs the HIP path (through the C ABI binding) for tests."""
from __future__ import annotations

import sys

import numpy as np
import torch

from workloads.generate import descriptor_arrays


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def api():
    import block_sparse_attention_pack_amd as P
    return P.api


def build_map(ps, block_m, block_n):
    A = api()
    P, R = descriptor_arrays(ps)
    pd, rd = A.descriptors_to_device(P, R)
    return A.pack_block_map(pd, rd, ps.B, ps.S, block_m, block_n)


def run_fwd_bwd(w, bwd=True):
    """Forward (and backward) of workload `w` on cuda:0; results on the CPU."""
    A = api()
    dev = "cuda"
    q, k, v, do = (x.to(dev).contiguous() for x in (w.q, w.k, w.v, w.do))
    fm = build_map(w.packset, *A.fwd_tile(w.Hq, w.Hkv, w.D))
    o, lse = A.packed_attn_fwd(fm, q, k, v, w.scale)
    out = {"o": o, "lse": lse, "fmap": fm}
    if bwd:
        bm = build_map(w.packset, *A.bwd_tile(w.Hq, w.Hkv, w.D))
        dq, dk, dv = A.packed_attn_bwd(fm, bm, q, k, v, o, lse, do, w.scale)
        out.update(dq=dq, dk=dk, dv=dv, bmap=bm)
    torch.cuda.synchronize()
    st = fm.status().cpu().tolist()
    assert st == [0, -1], st
    return {k_: (v_.cpu() if isinstance(v_, torch.Tensor) else v_) for k_, v_ in out.items()}


def rel_l2(x, ref):
    x = x.to(torch.float64)
    ref = ref.to(torch.float64)
    return float((x - ref).norm() / ref.norm().clamp_min(1e-300))
