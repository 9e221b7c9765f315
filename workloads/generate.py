"""Seeded generators for the five attention workloads and their variants.

Config numbering (1..5):
  1 tiny        batch 1, one pack prompt 64 + responses [32, 48], 2 q heads,
                2 kv heads, head_dim 64, unscaled N(0,1) values.
  2 qwen8b      8 rows, one [prompt|chosen|rejected] triple each, lognormal
                lengths; 32 q heads / 8 kv heads, head_dim 128.
  3 multirow    4 rows of 8192 tokens, greedy fill of lognormal triples.
  4 resplong    4 rows of prompt 256 + 2048 + 2048.
  5 group       2 rows, prompt 1024 shared by 8 responses of U[512, 1536].
Variant "3alt": rows of 56 fixed triples (64, [32, 48]) inside 8192 tokens.

The lengths stand in for the preference-data workloads the pages measured on
(UltraFeedback-family slices, p1 "UltraFeedback comparisons"): the lognormal
sigma 0.75 puts the capped mean response length near 375 tokens, inside the
338-416 / 364-405 averages p1 reports.  No dataset item is used.

RNG streams: lengths from numpy default_rng([cfg, seed, 0]); tensor values
from default_rng([cfg, seed, 1]), drawn in the order Q, K, V, dO as float32
standard normals, then rounded to bf16 (round to nearest even).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

CONFIG_NAMES = {1: "tiny", 2: "qwen3_8b_packs", 3: "multi_triple_rows",
                4: "response_long", 5: "group_pack", "3alt": "multi_triple_rows_fixed"}

_SIGMA = 0.75


@dataclass(frozen=True)
class Pack:
    """One pack: a prompt then its responses, contiguous in row `row` from `start`."""
    row: int
    start: int
    prompt_len: int
    resp_lens: Tuple[int, ...]

    @property
    def length(self) -> int:
        return self.prompt_len + sum(self.resp_lens)


@dataclass
class PackSet:
    B: int
    S: int
    packs: List[Pack] = field(default_factory=list)

    def real_tokens(self) -> int:
        return sum(p.length for p in self.packs)


@dataclass
class Workload:
    cfg: object
    seed: int
    packset: PackSet
    Hq: int
    Hkv: int
    D: int
    scale: float
    q: torch.Tensor   # bf16 [B, S, Hq, D]  (CPU)
    k: torch.Tensor   # bf16 [B, S, Hkv, D]
    v: torch.Tensor   # bf16 [B, S, Hkv, D]
    do: torch.Tensor  # bf16 [B, S, Hq, D]
    name: str = ""


def lognormal_length(rng: np.random.Generator, median: float, cap: int) -> int:
    z = rng.standard_normal()
    return int(min(cap, max(1, math.floor(math.exp(math.log(median) + _SIGMA * z) + 0.5))))


def _draw_triple(rng: np.random.Generator) -> Tuple[int, Tuple[int, int]]:
    p = lognormal_length(rng, 600, 2048)
    c = lognormal_length(rng, 300, 1024)
    r = lognormal_length(rng, 300, 1024)
    return p, (c, r)


def make_packset(cfg, seed: int = 0) -> PackSet:
    """Pack descriptors of config `cfg` (1..5 or "3alt")."""
    if cfg == 1:
        return PackSet(1, 144, [Pack(0, 0, 64, (32, 48))])
    if cfg == 2:
        rng = np.random.default_rng([2, seed, 0])
        trip = [_draw_triple(rng) for _ in range(8)]
        S = max(p + sum(rs) for p, rs in trip)
        return PackSet(8, S, [Pack(b, 0, p, rs) for b, (p, rs) in enumerate(trip)])
    if cfg == 3:
        rng = np.random.default_rng([3, seed, 0])
        B, S = 4, 8192
        packs = []
        for b in range(B):
            used = 0
            while True:
                p, rs = _draw_triple(rng)
                n = p + sum(rs)
                if used + n > S:
                    break
                packs.append(Pack(b, used, p, rs))
                used += n
        return PackSet(B, S, packs)
    if cfg == "3alt":
        B, S = 4, 8192
        packs = [Pack(b, t * 144, 64, (32, 48)) for b in range(B) for t in range(56)]
        return PackSet(B, S, packs)
    if cfg == 4:
        return PackSet(4, 4352, [Pack(b, 0, 256, (2048, 2048)) for b in range(4)])
    if cfg == 5:
        rng = np.random.default_rng([5, seed, 0])
        rows = [tuple(int(x) for x in rng.integers(512, 1537, size=8)) for _ in range(2)]
        S = max(1024 + sum(r) for r in rows)
        return PackSet(2, S, [Pack(b, 0, 1024, r) for b, r in enumerate(rows)])
    raise ValueError(f"unknown config {cfg!r}")


def _heads(cfg):
    if cfg == 1:
        return 2, 2, 64
    return 32, 8, 128


def _cfg_id(cfg) -> int:
    return 6 if cfg == "3alt" else int(cfg)


def _draw_tensors(rng, B, S, Hq, Hkv, D, qkv_scale: Optional[float]):
    q = rng.standard_normal((B, S, Hq, D), dtype=np.float32)
    k = rng.standard_normal((B, S, Hkv, D), dtype=np.float32)
    v = rng.standard_normal((B, S, Hkv, D), dtype=np.float32)
    do = rng.standard_normal((B, S, Hq, D), dtype=np.float32)
    if qkv_scale is not None:
        s = np.float32(qkv_scale)
        q *= s
        k *= s
        v *= s
    cast = lambda x: torch.from_numpy(x).to(torch.bfloat16)  # noqa: E731
    return cast(q), cast(k), cast(v), cast(do)


def make_workload(cfg, seed: int = 0, unscaled: bool = False,
                  packset: Optional[PackSet] = None,
                  heads: Optional[Tuple[int, int, int]] = None) -> Workload:
    """Descriptors plus seeded bf16 Q, K, V, dO for config `cfg`.

    Configs 2..5 multiply Q, K, V by 1/sqrt(128) before the bf16 cast unless
    `unscaled`; dO is never scaled.  `packset` / `heads` override the config's
    own (used for small custom cases); the softmax scale is 1/sqrt(D).
    """
    ps = packset if packset is not None else make_packset(cfg, seed)
    Hq, Hkv, D = heads if heads is not None else _heads(cfg)
    rng = np.random.default_rng([_cfg_id(cfg) if cfg is not None else 0, seed, 1])
    scaled = (cfg not in (1, None)) and not unscaled
    q, k, v, do = _draw_tensors(rng, ps.B, ps.S, Hq, Hkv, D,
                                (1.0 / math.sqrt(128.0)) if scaled else None)
    name = CONFIG_NAMES.get(cfg, "custom") if cfg is not None else "custom"
    return Workload(cfg, seed, ps, Hq, Hkv, D, 1.0 / math.sqrt(D), q, k, v, do,
                    name + ("_unscaled" if unscaled else ""))


def random_packset(rng: np.random.Generator, B: int, S: int, max_packs_per_row: int = 4,
                   max_resp: int = 4, max_len: int = 40, allow_zero: bool = True) -> PackSet:
    """Random ragged pack layout (zero-length prompts/responses and pad allowed)."""
    packs = []
    lo = 0 if allow_zero else 1
    for b in range(B):
        pos = int(rng.integers(0, 3))
        for _ in range(int(rng.integers(0, max_packs_per_row + 1))):
            p = int(rng.integers(lo, max_len + 1))
            rs = tuple(int(rng.integers(lo, max_len + 1)) for _ in range(int(rng.integers(0, max_resp + 1))))
            n = p + sum(rs)
            if pos + n > S:
                break
            packs.append(Pack(b, pos, p, rs))
            pos += n + int(rng.integers(0, 3))
    return PackSet(B, S, packs)


def descriptor_arrays(ps: PackSet) -> Tuple[np.ndarray, np.ndarray]:
    """Flat int32 descriptor table [P, 5] = (row, start, prompt_len, n_resp,
    resp_first) and the concatenated response lengths [R]."""
    rows, lens = [], []
    for p in ps.packs:
        rows.append((p.row, p.start, p.prompt_len, len(p.resp_lens), len(lens)))
        lens.extend(p.resp_lens)
    packs = np.asarray(rows, dtype=np.int32).reshape(-1, 5)
    return packs, np.asarray(lens, dtype=np.int32)


def pairwise_packset(ps: PackSet) -> Tuple[PackSet, List[Tuple[int, int, int, int]]]:
    """The vanilla pairwise layout: one row [prompt | response_k] per (pack, k).

    Returns the new pack set (one single-response pack per row, padded to the
    longest pair) and, per new row, (src_row, prompt_start, prompt_len,
    resp_start, resp_len) as a list of tuples for copying tensors.
    """
    pairs = []
    for p in ps.packs:
        off = p.start + p.prompt_len
        for r in p.resp_lens:
            pairs.append((p.row, p.start, p.prompt_len, off, r))
            off += r
    S2 = max((pl + r for _, _, pl, _, r in pairs), default=1)
    packs = [Pack(i, 0, pl, (r,)) for i, (_, _, pl, _, r) in enumerate(pairs)]
    return PackSet(len(pairs), S2, packs), pairs


def pairwise_tensors(x: torch.Tensor, pairs, S2: int) -> torch.Tensor:
    """Copy [B, S, H, D] rows into the pairwise layout [len(pairs), S2, H, D] (pad = 0)."""
    out = torch.zeros((len(pairs), S2) + tuple(x.shape[2:]), dtype=x.dtype, device=x.device)
    for i, (b, ps_, pl, rs_, rl) in enumerate(pairs):
        out[i, :pl] = x[b, ps_:ps_ + pl]
        out[i, pl:pl + rl] = x[b, rs_:rs_ + rl]
    return out


def pad_to_len(ps: PackSet, S_new: int) -> PackSet:
    """Same packs inside longer rows (extra tokens are pad)."""
    assert S_new >= ps.S
    return PackSet(ps.B, S_new, list(ps.packs))
