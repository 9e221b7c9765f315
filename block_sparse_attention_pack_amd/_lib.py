"""ctypes binding of libpba.so: argument marshalling only.

Torch tensors supply device memory and the current HIP stream; every step
of the computation runs in the library's kernels.  Importing this module
fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpba.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m block_sparse_attention_pack_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

PBA_OK = 0
TILE_SKIP, TILE_PARTIAL, TILE_FULL = 0, 1, 2
EXPORTED = ("pba_strerror", "pba_fwd_tile", "pba_bwd_tile", "pba_map_bytes", "pba_map_init",
            "pba_pack_block_map", "pba_pack_block_maps", "pba_packed_attn_fwd", "pba_bwd_workspace_bytes", "pba_packed_attn_bwd",
            "pba_packed_attn_bwd_stages", "pba_mfma_probe", "pba_lds_probe", "pba_valu_probe", "pba_pack_positions",
            "pba_packed_token_logp", "pba_group_coefficients", "pba_packed_rope", "pba_packed_attn_bwd_rope",
            "pba_packed_attn_fwd_rope", "pba_set_bwd_split_slots", "pba_packed_attn_bwd_noalloc")


class PbaBlockMap(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("S", ctypes.c_int32), ("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32),
        ("nqt", ctypes.c_int32), ("nkt", ctypes.c_int32),
        ("tok_pack", ctypes.c_void_p), ("tok_branch", ctypes.c_void_p), ("tok_win", ctypes.c_void_p),
        ("cls", ctypes.c_void_p), ("q2k_cnt", ctypes.c_void_p), ("q2k_idx", ctypes.c_void_p),
        ("k2q_cnt", ctypes.c_void_p), ("k2q_idx", ctypes.c_void_p), ("totals", ctypes.c_void_p),
        ("status", ctypes.c_void_p), ("q_order", ctypes.c_void_p), ("k_order", ctypes.c_void_p),
        ("work", ctypes.c_void_p),
    ]


_c_int_p = ctypes.POINTER(ctypes.c_int)
_lib.pba_strerror.argtypes = [ctypes.c_int]
_lib.pba_strerror.restype = ctypes.c_char_p
for _n in ("pba_fwd_tile", "pba_bwd_tile"):
    getattr(_lib, _n).argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _c_int_p, _c_int_p]
    getattr(_lib, _n).restype = ctypes.c_int
_lib.pba_map_bytes.argtypes = [ctypes.c_int] * 4
_lib.pba_map_bytes.restype = ctypes.c_size_t
_lib.pba_map_init.argtypes = [ctypes.POINTER(PbaBlockMap), ctypes.c_void_p, ctypes.c_size_t] + [ctypes.c_int] * 4
_lib.pba_map_init.restype = ctypes.c_int
_lib.pba_pack_block_map.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.POINTER(PbaBlockMap), ctypes.c_void_p]
_lib.pba_pack_block_map.restype = ctypes.c_int
_lib.pba_pack_block_maps.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                     ctypes.POINTER(PbaBlockMap), ctypes.c_int, ctypes.c_void_p]
_lib.pba_pack_block_maps.restype = ctypes.c_int
MAX_MAPS_PER_BUILD = 4
_lib.pba_packed_attn_fwd.argtypes = [ctypes.POINTER(PbaBlockMap)] + [ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + \
    [ctypes.c_float, ctypes.c_void_p]
_lib.pba_packed_attn_fwd.restype = ctypes.c_int
_lib.pba_bwd_workspace_bytes.argtypes = [ctypes.c_int] * 4
_lib.pba_bwd_workspace_bytes.restype = ctypes.c_size_t
_lib.pba_packed_attn_bwd.argtypes = [ctypes.POINTER(PbaBlockMap)] * 2 + [ctypes.c_void_p] * 10 + [ctypes.c_size_t] + \
    [ctypes.c_int] * 5 + [ctypes.c_float, ctypes.c_void_p]
_lib.pba_packed_attn_bwd.restype = ctypes.c_int
_lib.pba_packed_attn_bwd_stages.argtypes = [ctypes.c_int] + list(_lib.pba_packed_attn_bwd.argtypes)
_lib.pba_packed_attn_bwd_stages.restype = ctypes.c_int
_lib.pba_pack_positions.argtypes = [ctypes.POINTER(PbaBlockMap)] + [ctypes.c_void_p] * 4
_lib.pba_pack_positions.restype = ctypes.c_int
_lib.pba_packed_token_logp.argtypes = [ctypes.POINTER(PbaBlockMap), ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
_lib.pba_packed_token_logp.restype = ctypes.c_int
_lib.pba_group_coefficients.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_float, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
_lib.pba_group_coefficients.restype = ctypes.c_int
_lib.pba_packed_rope.argtypes = [ctypes.POINTER(PbaBlockMap), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
_lib.pba_packed_rope.restype = ctypes.c_int
_lib.pba_packed_attn_bwd_rope.argtypes = list(_lib.pba_packed_attn_bwd.argtypes[:-2]) + [ctypes.c_float, ctypes.c_float,
                                                                                        ctypes.c_void_p]
_lib.pba_packed_attn_bwd_rope.restype = ctypes.c_int
_lib.pba_packed_attn_fwd_rope.argtypes = [ctypes.POINTER(PbaBlockMap)] + [ctypes.c_void_p] * 6 + [ctypes.c_int] * 5 + \
    [ctypes.c_float, ctypes.c_float, ctypes.c_void_p]
_lib.pba_packed_attn_fwd_rope.restype = ctypes.c_int
_lib.pba_mfma_probe.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
_lib.pba_mfma_probe.restype = ctypes.c_int
_lib.pba_lds_probe.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
_lib.pba_lds_probe.restype = ctypes.c_int
_lib.pba_valu_probe.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
_lib.pba_valu_probe.restype = ctypes.c_int
_lib.pba_packed_attn_bwd_noalloc.argtypes = [ctypes.POINTER(PbaBlockMap)] * 2 + [ctypes.c_void_p] * 9 + \
    [ctypes.c_int] * 5 + [ctypes.c_float, ctypes.c_void_p]
_lib.pba_packed_attn_bwd_noalloc.restype = ctypes.c_int
NOALLOC_SCRATCH_BYTES = 96 << 20
_lib.pba_set_bwd_split_slots.argtypes = [ctypes.c_int]
_lib.pba_set_bwd_split_slots.restype = ctypes.c_int
BWD_DQ, BWD_DKDV, BWD_ALL = 1, 2, 3


class PbaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


def strerror(code: int) -> str:
    return _lib.pba_strerror(int(code)).decode()


def _check(rc: int, where: str):
    if rc != PBA_OK:
        raise PbaError(rc, where)


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def fwd_tile(Hq: int, Hkv: int, D: int) -> Tuple[int, int]:
    bm, bn = ctypes.c_int(), ctypes.c_int()
    _check(_lib.pba_fwd_tile(Hq, Hkv, D, ctypes.byref(bm), ctypes.byref(bn)), "pba_fwd_tile")
    return bm.value, bn.value


def bwd_tile(Hq: int, Hkv: int, D: int) -> Tuple[int, int]:
    bm, bn = ctypes.c_int(), ctypes.c_int()
    _check(_lib.pba_bwd_tile(Hq, Hkv, D, ctypes.byref(bm), ctypes.byref(bn)), "pba_bwd_tile")
    return bm.value, bn.value


def map_bytes(B: int, S: int, block_m: int, block_n: int) -> int:
    return int(_lib.pba_map_bytes(B, S, block_m, block_n))


def workspace_bytes(B: int, S: int, Hq: int, D: int) -> int:
    return int(_lib.pba_bwd_workspace_bytes(B, S, Hq, D))


class BlockMap:
    """A device block map: one torch uint8 buffer carved by pba_map_init."""

    def __init__(self, B: int, S: int, block_m: int, block_n: int, device="cuda",
                 buffer: Optional[torch.Tensor] = None):
        """buffer: optional caller-owned uint8 device tensor of at least
        map_bytes(...) bytes from its first 256-byte aligned address on (a
        fresh one of map_bytes + 256 bytes otherwise)."""
        nbytes = map_bytes(B, S, block_m, block_n)
        if nbytes == 0:
            raise PbaError(-2, "pba_map_bytes")
        if buffer is None:
            buffer = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        elif (buffer.dtype != torch.uint8 or not buffer.is_cuda or not buffer.is_contiguous()
              or buffer.numel() - (-buffer.data_ptr()) % 256 < nbytes):
            raise ValueError(f"map buffer must be a contiguous uint8 device tensor of {nbytes} bytes after alignment")
        self.buffer = buffer
        base = self.buffer.data_ptr()
        self._off0 = (-base) % 256
        self.struct = PbaBlockMap()
        _check(_lib.pba_map_init(ctypes.byref(self.struct), base + self._off0, nbytes, B, S, block_m, block_n),
               "pba_map_init")
        self.B, self.S, self.block_m, self.block_n = B, S, block_m, block_n
        self.nqt, self.nkt = self.struct.nqt, self.struct.nkt

    def _view(self, field: str, n: int, dtype) -> torch.Tensor:
        off = getattr(self.struct, field) - self.buffer.data_ptr()
        esz = torch.empty((), dtype=dtype).element_size()
        return self.buffer[off:off + n * esz].view(dtype)

    # Views of the map fields (device tensors), shaped like their definitions.
    def tok_pack(self):
        return self._view("tok_pack", self.B * self.S, torch.int32).view(self.B, self.S)

    def tok_branch(self):
        return self._view("tok_branch", self.B * self.S, torch.int32).view(self.B, self.S)

    def tok_win(self):
        return self._view("tok_win", self.B * self.S * 4, torch.int32).view(self.B, self.S, 4)

    def cls(self):
        return self._view("cls", self.B * self.nqt * self.nkt, torch.uint8).view(self.B, self.nqt, self.nkt)

    def q2k_cnt(self):
        return self._view("q2k_cnt", self.B * self.nqt * 2, torch.int32).view(self.B, self.nqt, 2)

    def q2k_idx(self):
        return self._view("q2k_idx", self.B * self.nqt * self.nkt, torch.int32).view(self.B, self.nqt, self.nkt)

    def k2q_cnt(self):
        return self._view("k2q_cnt", self.B * self.nkt * 2, torch.int32).view(self.B, self.nkt, 2)

    def k2q_idx(self):
        return self._view("k2q_idx", self.B * self.nkt * self.nqt, torch.int32).view(self.B, self.nkt, self.nqt)

    def totals(self):
        return self._view("totals", 3, torch.int64)

    def status(self):
        return self._view("status", 2, torch.int32)

    def q_order(self):
        return self._view("q_order", self.B * self.nqt, torch.int32)

    def k_order(self):
        return self._view("k_order", self.B * self.nkt, torch.int32)

    def to_host(self) -> dict:
        """Every field as numpy (synchronises)."""
        return {
            "B": self.B, "S": self.S, "block_m": self.block_m, "block_n": self.block_n,
            "nqt": self.nqt, "nkt": self.nkt,
            "tok_pack": self.tok_pack().cpu().numpy(), "tok_branch": self.tok_branch().cpu().numpy(),
            "tok_win": self.tok_win().cpu().numpy(), "cls": self.cls().cpu().numpy(),
            "q2k_cnt": self.q2k_cnt().cpu().numpy(), "q2k_idx": self.q2k_idx().cpu().numpy(),
            "k2q_cnt": self.k2q_cnt().cpu().numpy(), "k2q_idx": self.k2q_idx().cpu().numpy(),
            "totals": self.totals().cpu().numpy(), "status": self.status().cpu().numpy(),
            "q_order": self.q_order().cpu().numpy(), "k_order": self.k_order().cpu().numpy(),
        }


def descriptors_to_device(packs, resp_len, device="cuda") -> Tuple[torch.Tensor, torch.Tensor]:
    """int32 [P, 5] descriptor table and [R] response lengths as device tensors."""
    p = torch.as_tensor(packs, dtype=torch.int32).reshape(-1, 5).contiguous().to(device)
    r = torch.as_tensor(resp_len, dtype=torch.int32).reshape(-1).contiguous().to(device)
    return p, r


def _descriptors(packs_dev, resp_len_dev):
    _tensor(packs_dev, "packs", None, torch.int32, align=4)
    if packs_dev.numel() and (packs_dev.dim() != 2 or packs_dev.shape[1] != 5):
        raise ValueError(f"packs must be int32 [P, 5], got {tuple(packs_dev.shape)}")
    _tensor(resp_len_dev, "resp_len", (resp_len_dev.numel(),) if isinstance(resp_len_dev, torch.Tensor) else None,
            torch.int32, packs_dev.device, align=4)


def pack_block_map(packs_dev: torch.Tensor, resp_len_dev: torch.Tensor, B: int, S: int, block_m: int, block_n: int,
                   out: Optional[BlockMap] = None, stream=None) -> BlockMap:
    """pba_pack_block_map on device descriptors (int32 [P, 5] and [R])."""
    _descriptors(packs_dev, resp_len_dev)
    m = out if out is not None else BlockMap(B, S, block_m, block_n, device=packs_dev.device)
    _map(m, "out", B, S, packs_dev.device)
    if (m.block_m, m.block_n) != (block_m, block_n):
        raise ValueError(f"out was carved for tiles {m.block_m}x{m.block_n}, not {block_m}x{block_n}")
    n_packs = packs_dev.shape[0] if packs_dev.numel() else 0
    n_resp = resp_len_dev.numel()
    _check(_lib.pba_pack_block_map(packs_dev.data_ptr() if n_packs else None, n_packs,
                                   resp_len_dev.data_ptr() if n_resp else None, n_resp,
                                   ctypes.byref(m.struct), _stream(stream)), "pba_pack_block_map")
    return m


def pack_block_maps(packs_dev: torch.Tensor, resp_len_dev: torch.Tensor, maps: Sequence[BlockMap],
                    stream=None) -> Sequence[BlockMap]:
    """pba_pack_block_maps: build several maps of the same (B, S) together."""
    if not 1 <= len(maps) <= MAX_MAPS_PER_BUILD:
        raise ValueError(f"1 to {MAX_MAPS_PER_BUILD} maps per build")
    _descriptors(packs_dev, resp_len_dev)
    for i, m in enumerate(maps):
        _map(m, f"maps[{i}]", maps[0].B, maps[0].S, packs_dev.device)
    arr = (PbaBlockMap * len(maps))(*[m.struct for m in maps])
    n_packs = packs_dev.shape[0] if packs_dev.numel() else 0
    n_resp = resp_len_dev.numel()
    _check(_lib.pba_pack_block_maps(packs_dev.data_ptr() if n_packs else None, n_packs,
                                    resp_len_dev.data_ptr() if n_resp else None, n_resp, arr, len(maps),
                                    _stream(stream)), "pba_pack_block_maps")
    return maps


def _tensor(x, name: str, shape=None, dtype=torch.bfloat16, device=None, align: int = 16):
    """Reject, before any pointer reaches the library, a tensor that is not a
    contiguous device tensor of the expected dtype, shape and device (a
    mismatch would otherwise become out-of-bounds device accesses)."""
    if not isinstance(x, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor, got {type(x).__name__}")
    if x.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {x.dtype}")
    if not x.is_cuda:
        raise ValueError(f"{name} must be a device (cuda) tensor, got one on {x.device}")
    if device is not None and x.device != device:
        raise ValueError(f"{name} is on {x.device}, the other operands on {device}")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(x.shape)}, expected {tuple(shape)}")
    if x.numel() and x.data_ptr() % align:
        raise ValueError(f"{name} must be {align}-byte aligned")


def _disjoint(outputs: dict, inputs: dict):
    """Reject outputs whose memory overlaps an input or another output (the
    kernels read inputs while other workgroups write outputs)."""
    def span(t):
        n = t.numel() * t.element_size()
        return (t.data_ptr(), t.data_ptr() + n) if n else None
    outs = [(k, span(t)) for k, t in outputs.items()]
    ins = [(k, span(t)) for k, t in inputs.items()]
    for i, (name, a) in enumerate(outs):
        if a is None:
            continue
        for other, b in ins + outs[i + 1:]:
            if b is not None and a[0] < b[1] and b[0] < a[1]:
                raise ValueError(f"{name} overlaps {other} in memory")


def _bf16(x, name: str, shape=None, device=None):
    _tensor(x, name, shape, torch.bfloat16, device)


def _qkv(q, k, v, qname="q", kname="k"):
    """(B, S, Hq, Hkv, D) of bf16 q [B, S, Hq, D] and k, v [B, S, Hkv, D]."""
    _bf16(q, qname)
    if q.dim() != 4:
        raise ValueError(f"{qname} must be [B, S, Hq, D], got shape {tuple(q.shape)}")
    B, S, Hq, D = q.shape
    _bf16(k, kname, device=q.device)
    if k.dim() != 4 or (k.shape[0], k.shape[1], k.shape[3]) != (B, S, D):
        raise ValueError(f"{kname} must be [B, S, Hkv, D] = [{B}, {S}, Hkv, {D}], got {tuple(k.shape)}")
    Hkv = k.shape[2]
    _bf16(v, "v", k.shape, q.device)
    return B, S, Hq, Hkv, D


def _map(m, name: str, B: int, S: int, device):
    if not isinstance(m, BlockMap):
        raise ValueError(f"{name} must be a BlockMap")
    if (m.B, m.S) != (B, S):
        raise ValueError(f"{name} was built for (B, S) = ({m.B}, {m.S}), the tensors are ({B}, {S})")
    if m.buffer.device != device:
        raise ValueError(f"{name} lives on {m.buffer.device}, the tensors on {device}")


def _workspace(ws, need: int, device):
    """(256-byte aligned address, usable bytes) of a caller workspace."""
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    if ws.device != device:
        raise ValueError(f"workspace is on {ws.device}, the tensors on {device}")
    base = ws.data_ptr()
    off = (-base) % 256
    nbytes = ws.numel() * ws.element_size() - off
    if nbytes < need:
        raise ValueError(f"workspace holds {nbytes} usable bytes after 256-byte alignment, needs {need}")
    return base + off, nbytes


def packed_attn_fwd(m: BlockMap, q, k, v, softmax_scale: Optional[float] = None,
                    out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None, stream=None):
    """O [B, S, Hq, D] bf16 and LSE [B, Hq, S] fp32."""
    B, S, Hq, Hkv, D = _qkv(q, k, v)
    _map(m, "map", B, S, q.device)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _bf16(o, "o", q.shape, q.device)
        _tensor(lse, "lse", (B, Hq, S), torch.float32, q.device, align=4)
        _disjoint({"o": o, "lse": lse}, {"q": q, "k": k, "v": v})
    _check(_lib.pba_packed_attn_fwd(ctypes.byref(m.struct), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                    lse.data_ptr(), B, S, Hq, Hkv, D, scale, _stream(stream)), "pba_packed_attn_fwd")
    return o, lse


def _bwd_operands(qmap, kmap, q, k, v, o, lse, dout, out, workspace, qname="q", kname="k"):
    B, S, Hq, Hkv, D = _qkv(q, k, v, qname, kname)
    _map(qmap, "qmap", B, S, q.device)
    _map(kmap, "kmap", B, S, q.device)
    _bf16(o, "o", q.shape, q.device)
    _bf16(dout, "dout", q.shape, q.device)
    _tensor(lse, "lse", (B, Hq, S), torch.float32, q.device, align=4)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
        _bf16(dq, "dq", q.shape, q.device)
        _bf16(dk, "dk", k.shape, q.device)
        _bf16(dv, "dv", k.shape, q.device)
    need = workspace_bytes(B, S, Hq, D)
    if workspace is None:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=q.device)
    ws, ws_bytes = _workspace(workspace, need, q.device)
    _disjoint({"dq": dq, "dk": dk, "dv": dv, "workspace": workspace},
              {qname: q, kname: k, "v": v, "o": o, "lse": lse, "dout": dout})
    return (B, S, Hq, Hkv, D), (dq, dk, dv), ws, ws_bytes


def packed_attn_bwd(qmap: BlockMap, kmap: BlockMap, q, k, v, o, lse, dout, softmax_scale: Optional[float] = None,
                    out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None, stages: int = BWD_ALL):
    """dQ, dK, dV (bf16) for the loss <dO, O>.  qmap has the forward's tile
    shape (fwd_tile), kmap the backward's (bwd_tile).  `stages` selects a
    subset of the backward's stages (BWD_DQ | BWD_DKDV)."""
    (B, S, Hq, Hkv, D), (dq, dk, dv), ws, ws_bytes = _bwd_operands(qmap, kmap, q, k, v, o, lse, dout, out, workspace)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    _check(_lib.pba_packed_attn_bwd_stages(stages, ctypes.byref(qmap.struct), ctypes.byref(kmap.struct), q.data_ptr(),
                                           k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                                           dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws, ws_bytes, B, S, Hq, Hkv,
                                           D, scale, _stream(stream)),
           "pba_packed_attn_bwd_stages")
    return dq, dk, dv


def packed_attn_bwd_noalloc(qmap: BlockMap, kmap: BlockMap, q, k, v, o, lse, dout,
                            softmax_scale: Optional[float] = None,
                            out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None, stream=None):
    """packed_attn_bwd through pba_packed_attn_bwd_noalloc: the library's own
    device scratch instead of a workspace (the C call allocates nothing; pass
    `out` to keep this wrapper from allocating the outputs)."""
    B, S, Hq, Hkv, D = _qkv(q, k, v)
    _map(qmap, "qmap", B, S, q.device)
    _map(kmap, "kmap", B, S, q.device)
    _bf16(o, "o", q.shape, q.device)
    _bf16(dout, "dout", q.shape, q.device)
    _tensor(lse, "lse", (B, Hq, S), torch.float32, q.device, align=4)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
        _bf16(dq, "dq", q.shape, q.device)
        _bf16(dk, "dk", k.shape, q.device)
        _bf16(dv, "dv", k.shape, q.device)
        _disjoint({"dq": dq, "dk": dk, "dv": dv}, {"q": q, "k": k, "v": v, "o": o, "lse": lse, "dout": dout})
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    _check(_lib.pba_packed_attn_bwd_noalloc(ctypes.byref(qmap.struct), ctypes.byref(kmap.struct), q.data_ptr(),
                                            k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                                            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, S, Hq, Hkv, D, scale,
                                            _stream(stream)),
           "pba_packed_attn_bwd_noalloc")
    return dq, dk, dv


def set_bwd_split_slots(slots: int) -> int:
    """Fix the workgroup slots per kv group of the dK / dV split rule for the
    process (0 = the device's compute units / Hkv, the default); returns the
    previous setting.  Which key tiles are split sets the rounding of their
    dK / dV, so fixing it makes results independent of the device's CU count."""
    rc = _lib.pba_set_bwd_split_slots(int(slots))
    if rc < 0:
        raise PbaError(rc, "pba_set_bwd_split_slots")
    return rc


def packed_attn_fwd_rope(m: BlockMap, q, k_rot, v, rope_base: float, softmax_scale: Optional[float] = None,
                         out=None, q_rot_out=True, stream=None):
    """(o, lse, q_rot): forward for rotary inputs with Q's rotation fused in
    (q unrotated, k_rot from packed_rope).  q_rot_out: True to allocate the
    rotated Q the kernel writes for the backward, a tensor to write it
    there, or None/False not to write it."""
    B, S, Hq, Hkv, D = _qkv(q, k_rot, v, "q", "k_rot")
    _map(m, "map", B, S, q.device)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _bf16(o, "o", q.shape, q.device)
        _tensor(lse, "lse", (B, Hq, S), torch.float32, q.device, align=4)
    if q_rot_out is True:
        q_rot = torch.empty_like(q)
    elif q_rot_out is None or q_rot_out is False:
        q_rot = None
    else:
        q_rot = q_rot_out
        _bf16(q_rot, "q_rot_out", q.shape, q.device)
    outs = {"o": o, "lse": lse}
    if q_rot is not None:
        outs["q_rot_out"] = q_rot
    _disjoint(outs, {"q": q, "k_rot": k_rot, "v": v})
    _check(_lib.pba_packed_attn_fwd_rope(ctypes.byref(m.struct), q.data_ptr(), k_rot.data_ptr(), v.data_ptr(),
                                         o.data_ptr(), lse.data_ptr(), None if q_rot is None else q_rot.data_ptr(),
                                         B, S, Hq, Hkv, D, scale, float(rope_base), _stream(stream)),
           "pba_packed_attn_fwd_rope")
    return o, lse, q_rot


def packed_attn_bwd_rope(qmap: BlockMap, kmap: BlockMap, q_rot, k_rot, v, o, lse, dout, rope_base: float,
                         softmax_scale: Optional[float] = None,
                         out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None):
    """dQ, dK (with respect to the unrotated Q and K) and dV for inputs
    rotated by packed_rope(..., rope_base): the inverse rotation of the
    gradients runs inside the backward kernels."""
    (B, S, Hq, Hkv, D), (dq, dk, dv), ws, ws_bytes = _bwd_operands(qmap, kmap, q_rot, k_rot, v, o, lse, dout, out,
                                                                   workspace, "q_rot", "k_rot")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    _check(_lib.pba_packed_attn_bwd_rope(ctypes.byref(qmap.struct), ctypes.byref(kmap.struct), q_rot.data_ptr(),
                                         k_rot.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                                         dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws, ws_bytes, B, S, Hq, Hkv, D,
                                         scale, float(rope_base), _stream(stream)),
           "pba_packed_attn_bwd_rope")
    return dq, dk, dv


# FLOP of one pba_mfma_probe iteration per workgroup: 4 waves x 16 MFMAs x 32x32x16x2.
MFMA_PROBE_FLOP_PER_BLOCK_ITER = 4 * 16 * 32 * 32 * 16 * 2


def mfma_probe(out: torch.Tensor, n_blocks: int, iters: int, stream=None) -> None:
    """Enqueue the library's sustained-MFMA-rate loop (a measurement helper);
    `out` is a float32 device tensor of at least n_blocks * 256 elements."""
    if out.dtype != torch.float32 or out.numel() < n_blocks * 256 or not out.is_cuda:
        raise ValueError("out must be a float32 device tensor of n_blocks * 256 elements")
    _check(_lib.pba_mfma_probe(out.data_ptr(), n_blocks, iters, _stream(stream)), "pba_mfma_probe")


def lds_probe(out: torch.Tensor, n_blocks: int, iters: int, stream=None) -> None:
    """Enqueue the library's LDS read-bandwidth loop (a measurement helper);
    `out` is a float32 device tensor of at least n_blocks * 512 elements."""
    if out.dtype != torch.float32 or out.numel() < n_blocks * 512 or not out.is_cuda:
        raise ValueError("out must be a float32 device tensor of n_blocks * 512 elements")
    _check(_lib.pba_lds_probe(out.data_ptr(), n_blocks, iters, _stream(stream)), "pba_lds_probe")


def valu_probe(out: torch.Tensor, n_blocks: int, iters: int, exp2: bool, stream=None) -> None:
    """Enqueue the library's FMA (exp2=False) or exp2 + multiply (exp2=True)
    issue-rate loop; `out` is a float32 device tensor of n_blocks * 256."""
    if out.dtype != torch.float32 or out.numel() < n_blocks * 256 or not out.is_cuda:
        raise ValueError("out must be a float32 device tensor of n_blocks * 256 elements")
    _check(_lib.pba_valu_probe(out.data_ptr(), n_blocks, iters, int(bool(exp2)), _stream(stream)), "pba_valu_probe")


def pack_positions(m: BlockMap, out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None, stream=None):
    """(pos_ids int32 [B,S], src_row int32 [B,S], loss_mask uint8 [B,S]) of a
    built map: aligned positions, the row whose logits predict each token,
    and the response tokens that enter the log-prob sums."""
    dev = m.buffer.device
    if out is None:
        pos = torch.empty((m.B, m.S), dtype=torch.int32, device=dev)
        src = torch.empty((m.B, m.S), dtype=torch.int32, device=dev)
        mask = torch.empty((m.B, m.S), dtype=torch.uint8, device=dev)
    else:
        pos, src, mask = out
        for x, n, dt in ((pos, "pos_ids", torch.int32), (src, "src_row", torch.int32), (mask, "loss_mask", torch.uint8)):
            if x is not None:
                _tensor(x, n, (m.B, m.S), dt, dev, align=1)
    ptr = lambda x: None if x is None else x.data_ptr()  # noqa: E731
    _check(_lib.pba_pack_positions(ctypes.byref(m.struct), ptr(pos), ptr(src), ptr(mask), _stream(stream)),
           "pba_pack_positions")
    return pos, src, mask


def packed_token_logp(m: BlockMap, src_row, loss_mask, logits, tokens, packs_dev=None, resp_len_dev=None,
                      out: Optional[Tuple[torch.Tensor, Optional[torch.Tensor]]] = None, stream=None):
    """(tok_logp fp32 [B,S], resp_logp fp32 [n_resp] or None): log-softmax of
    each response token's predicting row at its token id, and the
    per-response sums (when the descriptors are given)."""
    _bf16(logits, "logits")
    if logits.dim() != 3:
        raise ValueError(f"logits must be bf16 [B, S, V], got shape {tuple(logits.shape)}")
    B, S, V = logits.shape
    dev = logits.device
    _map(m, "map", B, S, dev)
    _tensor(src_row, "src_row", (B, S), torch.int32, dev, align=4)
    _tensor(loss_mask, "loss_mask", (B, S), torch.uint8, dev, align=1)
    _tensor(tokens, "tokens", (B, S), torch.int32, dev, align=4)
    if (packs_dev is None) != (resp_len_dev is None):
        raise ValueError("give both packs_dev and resp_len_dev, or neither")
    if packs_dev is not None:
        _descriptors(packs_dev, resp_len_dev)
        if packs_dev.device != dev:
            raise ValueError("descriptors and logits are on different devices")
    if out is None:
        tok = torch.empty((B, S), dtype=torch.float32, device=dev)
        resp = None if packs_dev is None else torch.empty(resp_len_dev.numel(), dtype=torch.float32, device=dev)
    else:
        tok, resp = out
        _tensor(tok, "tok_logp", (B, S), torch.float32, dev, align=4)
        if resp is not None:
            if packs_dev is None:
                raise ValueError("resp_logp needs the descriptors")
            _tensor(resp, "resp_logp", (resp_len_dev.numel(),), torch.float32, dev, align=4)
    n_packs = 0 if packs_dev is None else packs_dev.shape[0]
    n_resp = 0 if resp_len_dev is None else resp_len_dev.numel()
    ptr = lambda x: None if x is None else x.data_ptr()  # noqa: E731
    _check(_lib.pba_packed_token_logp(ctypes.byref(m.struct), ptr(packs_dev), n_packs, ptr(resp_len_dev), n_resp,
                                      src_row.data_ptr(), loss_mask.data_ptr(), logits.data_ptr(), V,
                                      tokens.data_ptr(), tok.data_ptr(), ptr(resp), _stream(stream)),
           "pba_packed_token_logp")
    return tok, resp


GROUP_OBJECTIVES = {"all_pairs": 0, "margin": 1, "mpo": 2, "softmax": 3}
GROUP_MAX_ENTRIES = 4096


def groups_from_packs(n_resp_per_pack, positive):
    """CSR group arrays (group_ptr, member) with one group per pack, whose
    entries are that pack's responses in order; `positive` (one flag per
    response, packs in order) marks the preferred ones.  Host-side index
    bookkeeping only."""
    n = [int(x) for x in n_resp_per_pack]
    ptr = [0]
    for x in n:
        ptr.append(ptr[-1] + x)
    if len(positive) != ptr[-1]:
        raise ValueError("one positive flag per response")
    return (torch.tensor(ptr, dtype=torch.int32), torch.arange(ptr[-1], dtype=torch.int32),
            torch.as_tensor(positive, dtype=torch.uint8))


def group_coefficients(group_ptr, member, positive, pol, ref, resp_len, beta: float, objective="all_pairs",
                       alpha: float = 1.0, out=None, stream=None):
    """(coef fp32 [n_resp], nll_w fp32 [n_resp], loss fp32 [2], status int32
    [2]): surrogate coefficients of a group preference objective, the
    positive-NLL weights, (L_group, NLL term) and the device status, from
    device arrays (group_ptr int32 [G+1], member int32 / positive uint8
    [E], pol / ref fp32 and resp_len int32 [n_resp])."""
    obj = GROUP_OBJECTIVES[objective] if isinstance(objective, str) else int(objective)
    dev = pol.device if isinstance(pol, torch.Tensor) else None
    for t, n, dt in ((group_ptr, "group_ptr", torch.int32), (member, "member", torch.int32),
                     (positive, "positive", torch.uint8), (pol, "pol", torch.float32), (ref, "ref", torch.float32),
                     (resp_len, "resp_len", torch.int32)):
        _tensor(t, n, (t.numel(),) if isinstance(t, torch.Tensor) else None, dt, dev, align=1)
    n_resp = pol.numel()
    if ref.numel() != n_resp or resp_len.numel() != n_resp or positive.numel() != member.numel():
        raise ValueError("array sizes do not match")
    if group_ptr.numel() < 2:
        raise ValueError("group_ptr needs n_groups + 1 >= 2 entries")
    if out is None:
        out = (torch.empty(n_resp, dtype=torch.float32, device=dev), torch.empty(n_resp, dtype=torch.float32, device=dev),
               torch.empty(2, dtype=torch.float32, device=dev), torch.empty(2, dtype=torch.int32, device=dev))
    coef, nll_w, loss, status = out
    _tensor(coef, "coef", (n_resp,), torch.float32, dev, align=4)
    if nll_w is not None:
        _tensor(nll_w, "nll_w", (n_resp,), torch.float32, dev, align=4)
    if loss is not None:
        _tensor(loss, "loss", (2,), torch.float32, dev, align=4)
    _tensor(status, "status", (2,), torch.int32, dev, align=4)
    ptr = lambda x: None if x is None else x.data_ptr()  # noqa: E731
    _check(_lib.pba_group_coefficients(group_ptr.data_ptr(), group_ptr.numel() - 1, member.data_ptr(),
                                       positive.data_ptr(), member.numel(), pol.data_ptr(), ref.data_ptr(),
                                       resp_len.data_ptr(), n_resp, obj, float(beta), float(alpha), coef.data_ptr(),
                                       ptr(nll_w), ptr(loss), status.data_ptr(), _stream(stream)),
           "pba_group_coefficients")
    return coef, nll_w, loss, status


def packed_rope(m: BlockMap, x, base: float = 10000.0, inverse: bool = False, out=None, stream=None):
    """Rotary embedding of x (bf16 [B, S, H, D]) at the map's packed,
    branch-aligned position ids; inverse=True rotates back (for gradients).
    out may be x itself (in place)."""
    _bf16(x, "x")
    if x.dim() != 4:
        raise ValueError(f"x must be bf16 [B, S, H, D], got shape {tuple(x.shape)}")
    B, S, H, D = x.shape
    _map(m, "map", B, S, x.device)
    y = torch.empty_like(x) if out is None else out
    _bf16(y, "out", x.shape, x.device)
    _check(_lib.pba_packed_rope(ctypes.byref(m.struct), x.data_ptr(), y.data_ptr(), H, D, float(base),
                                int(bool(inverse)), _stream(stream)), "pba_packed_rope")
    return y
