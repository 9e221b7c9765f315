"""Runs the HIP path (through the C ABI binding) for tests.

Every output, workspace and map buffer handed to the library here sits
between two guard bands of a known byte pattern (the interior starts with
the same pattern, so an element the kernels fail to write shows up too);
`run_fwd_bwd` checks after the call that the bands are intact, so a store
past either end of a buffer fails the test that made it."""
from __future__ import annotations

import sys

import numpy as np
import torch

from workloads.generate import descriptor_arrays

GUARD_BYTES = 8192
GUARD_BYTE = 0xA5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def api():
    import block_sparse_attention_pack_amd as P
    return P.api


class Guarded:
    """nbytes of device memory between two GUARD_BYTES bands, all filled
    with GUARD_BYTE; the interior starts 256-byte aligned."""

    def __init__(self, nbytes: int, name: str, device="cuda"):
        self.name, self.n = name, int(nbytes)
        self.raw = torch.full((self.n + 2 * GUARD_BYTES + 256,), GUARD_BYTE, dtype=torch.uint8, device=device)
        self.lo = GUARD_BYTES + (-(self.raw.data_ptr() + GUARD_BYTES)) % 256
        self.hi = self.lo + self.n

    def bytes(self) -> torch.Tensor:
        return self.raw[self.lo:self.hi]

    def view(self, shape, dtype) -> torch.Tensor:
        return self.bytes().view(dtype).view(shape)

    def check(self):
        before = self.raw[self.lo - GUARD_BYTES:self.lo]
        after = self.raw[self.hi:self.hi + GUARD_BYTES]
        bad_lo = int((before != GUARD_BYTE).sum())
        bad_hi = int((after != GUARD_BYTE).sum())
        assert bad_lo == 0 and bad_hi == 0, f"{self.name}: guard bytes overwritten ({bad_lo} before, {bad_hi} after)"


def guarded_like(x: torch.Tensor, name: str, guards: list) -> torch.Tensor:
    g = Guarded(x.numel() * x.element_size(), name, x.device)
    guards.append(g)
    return g.view(x.shape, x.dtype)


def guarded_empty(shape, dtype, name: str, guards: list, device="cuda") -> torch.Tensor:
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    g = Guarded(n, name, device)
    guards.append(g)
    return g.view(shape, dtype)


def guarded_map(ps, block_m, block_n, guards: list):
    """A block map of ps built into a guard-banded buffer."""
    A = api()
    nbytes = A.map_bytes(ps.B, ps.S, block_m, block_n)
    g = Guarded(nbytes, f"map {block_m}x{block_n}")
    guards.append(g)
    m = A.BlockMap(ps.B, ps.S, block_m, block_n, buffer=g.bytes())
    P, R = descriptor_arrays(ps)
    pd, rd = A.descriptors_to_device(P, R)
    return A.pack_block_map(pd, rd, ps.B, ps.S, block_m, block_n, out=m)


def build_map(ps, block_m, block_n):
    A = api()
    P, R = descriptor_arrays(ps)
    pd, rd = A.descriptors_to_device(P, R)
    return A.pack_block_map(pd, rd, ps.B, ps.S, block_m, block_n)


def run_fwd_bwd(w, bwd=True):
    """Forward (and backward) of workload `w` on cuda:0; results on the CPU.
    Outputs, maps and the workspace are guard-banded and checked."""
    A = api()
    dev = "cuda"
    guards: list = []
    q, k, v, do = (x.to(dev).contiguous() for x in (w.q, w.k, w.v, w.do))
    fm = guarded_map(w.packset, *A.fwd_tile(w.Hq, w.Hkv, w.D), guards)
    o = guarded_like(q, "o", guards)
    lse = guarded_empty((w.packset.B, w.Hq, w.packset.S), torch.float32, "lse", guards)
    A.packed_attn_fwd(fm, q, k, v, w.scale, out=(o, lse))
    out = {"o": o, "lse": lse, "fmap": fm}
    if bwd:
        bm = guarded_map(w.packset, *A.bwd_tile(w.Hq, w.Hkv, w.D), guards)
        dq, dk, dv = guarded_like(q, "dq", guards), guarded_like(k, "dk", guards), guarded_like(v, "dv", guards)
        need = A.workspace_bytes(w.packset.B, w.packset.S, w.Hq, w.D)
        ws = Guarded(need, "workspace")
        guards.append(ws)
        A.packed_attn_bwd(fm, bm, q, k, v, o, lse, do, w.scale, out=(dq, dk, dv), workspace=ws.bytes())
        out.update(dq=dq, dk=dk, dv=dv, bmap=bm)
    torch.cuda.synchronize()
    st = fm.status().cpu().tolist()
    assert st == [0, -1], st
    for g in guards:
        g.check()
    return {k_: (v_.cpu() if isinstance(v_, torch.Tensor) else v_) for k_, v_ in out.items()}


def rel_l2(x, ref):
    x = x.to(torch.float64)
    ref = ref.to(torch.float64)
    return float((x - ref).norm() / ref.norm().clamp_min(1e-300))
