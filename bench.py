#!/usr/bin/env python3
"""Throughput of packed branch-aware attention (fwd + bwd) on one MI355X.

One step = the whole hot path over one batch: build the query-major and
key-major block maps from the pack descriptors, the forward kernel, then the
two backward kernels (dQ with rowsum(dO*O), then dK/dV).  Inputs are resident
in HBM before timing; outputs, maps and workspace are preallocated.

Metric: useful TFLOP/s = 14 * D * Hq * (allowed query-key pairs) per step /
step time (4*D forward + 10*D backward per allowed pair and q head; masked
pairs and skipped tiles earn nothing), also as a fraction of the bf16 MFMA
peak.  Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--config 2]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12   # 2516.6: 256 CUs x 2.4 GHz x 4096 bf16 FLOP/clk/CU (dense)
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_cfg(s):
    return s if s == "3alt" else int(s)


class Runner:
    """Preallocated buffers for one workload; step() enqueues the hot path."""

    def __init__(self, A, torch, ps, q, k, v, do, Hq, Hkv, D, scale, dense=False):
        from workloads.generate import descriptor_arrays
        self.A, self.torch = A, torch
        self.ps, self.Hq, self.Hkv, self.D, self.scale = ps, Hq, Hkv, D, scale
        P, R = descriptor_arrays(ps)
        self.P, self.R = A.descriptors_to_device(P, R)
        self.n_packs, self.n_resp = P.shape[0], R.shape[0]
        self.ftile, self.btile = A.fwd_tile(Hq, Hkv, D), A.bwd_tile(Hq, Hkv, D)
        self.fmap = A.BlockMap(ps.B, ps.S, *self.ftile)
        self.bmap = A.BlockMap(ps.B, ps.S, *self.btile)
        self.q, self.k, self.v, self.do = q, k, v, do
        self.o = torch.empty_like(q)
        self.lse = torch.empty((ps.B, Hq, ps.S), dtype=torch.float32, device=q.device)
        self.dq, self.dk, self.dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        self.ws = torch.empty(A.workspace_bytes(ps.B, ps.S, Hq, D) + 256, dtype=torch.uint8, device=q.device)
        self.dense = dense
        if dense:
            self.build_maps()
            for m in (self.fmap, self.bmap):
                self._densify(m)
            torch.cuda.synchronize()

    def _densify(self, m):
        """Every tile pair visited and masked: the dense packed baseline."""
        t = self.torch
        m.q2k_cnt()[:, :, 0] = 0
        m.q2k_cnt()[:, :, 1] = m.nkt
        m.q2k_idx().copy_(t.arange(m.nkt, dtype=t.int32, device="cuda").expand(m.B, m.nqt, m.nkt))
        m.k2q_cnt()[:, :, 0] = 0
        m.k2q_cnt()[:, :, 1] = m.nqt
        m.k2q_idx().copy_(t.arange(m.nqt, dtype=t.int32, device="cuda").expand(m.B, m.nkt, m.nqt))

    def build_maps(self):
        self.A.pack_block_maps(self.P, self.R, [self.fmap, self.bmap])

    def fwd(self):
        self.A.packed_attn_fwd(self.fmap, self.q, self.k, self.v, self.scale, out=(self.o, self.lse))

    def bwd(self, stages):
        self.A.packed_attn_bwd(self.fmap, self.bmap, self.q, self.k, self.v, self.o, self.lse, self.do, self.scale,
                               out=(self.dq, self.dk, self.dv), workspace=self.ws, stages=stages)

    def step(self, ev=None):
        A = self.A
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        if not self.dense:
            self.build_maps()
        rec(1)
        self.fwd()
        rec(2)
        self.bwd(A.BWD_DQ)
        rec(3)
        self.bwd(A.BWD_DKDV)
        rec(4)


def time_runner(torch, r, steps, warmup):
    for _ in range(warmup):
        r.step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        r.step(evs[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    names = ["map", "fwd", "bwd_dq", "bwd_dkdv"]
    per = {n: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / steps for i, n in enumerate(names)}
    per["step_events"] = sum(e[0].elapsed_time(e[4]) for e in evs) / steps
    return wall * 1e3, per


def allowed_pairs(ps):
    n = 0
    for p in ps.packs:
        n += p.prompt_len * (p.prompt_len + 1) // 2
        for r in p.resp_lens:
            n += r * p.prompt_len + r * (r + 1) // 2
    return n


def map_bytes(r, m):
    B, S = r.ps.B, r.ps.S
    return (20 * r.n_packs + 4 * r.n_resp + 24 * B * S + 9 * B * m.nqt * m.nkt + 12 * B * (m.nqt + m.nkt))


def sources_sha256(names):
    """sha256 over the named csrc files, in order (identifies a kernel build)."""
    h = hashlib.sha256()
    for n in names:
        h.update(open(os.path.join(ROOT, "block_sparse_attention_pack_amd", "csrc", n), "rb").read())
    return h.hexdigest()


def traffic_record(kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if sources_sha256(rec["sources"]) != rec.get("sources_sha256"):
        return None
    return rec


TRAFFIC_KERNELS = {  # record name -> (kernel name prefix in rocprofv3 output, source files)
    "fwd": ("fwd_kernel<128, 4, false>", ["pba_fwd.hip", "pba_tile.h", "pba_internal.h"]),
    "bwd_dq": ("bwd_dq<128, 4>", ["pba_bwd.hip", "pba_tile.h", "pba_internal.h"]),
    "bwd_dkdv": ("bwd_dkdv<128>", ["pba_bwd.hip", "pba_tile.h", "pba_internal.h"]),
}


def write_traffic(fetch_csv, write_csv, workload, out_dir=None):
    """profiles/traffic_<kernel>.json from two rocprofv3 --pmc runs of
    `bench.py --copy-calibration` (FETCH_SIZE, then WRITE_SIZE; KiB per
    dispatch), each scaled by what the same counter reads for the plain
    2^28-byte device copy (2^28 bytes read and written per launch)."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                name = row["Kernel_Name"]
                # The calibration copy is the only copy dispatch of 2^28 bytes
                # (its grid is far larger than the small descriptor copies').
                if "copyBuffer" in name:
                    if int(row["Grid_Size"]) < 65536:
                        continue
                    name = "calibration copyBuffer"
                vals.setdefault(name, []).append(float(row["Counter_Value"]))
        return vals

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")

    def avg(vals, prefix):
        xs = [x for name, v in vals.items() if prefix in name for x in v]
        if not xs:
            raise SystemExit(f"no {prefix} dispatches in the counter output")
        return sum(xs) / len(xs), len(xs)

    copy_kib = float(1 << 28) / 1024
    fetch_scale = copy_kib / avg(fetch, "calibration copyBuffer")[0]
    write_scale = copy_kib / avg(write, "calibration copyBuffer")[0]
    for rec_name, (prefix, sources) in TRAFFIC_KERNELS.items():
        fk, n = avg(fetch, prefix)
        wk, _ = avg(write, prefix)
        rec = {"kernel": rec_name, "workload": workload, "sources": sources,
               "sources_sha256": sources_sha256(sources), "dispatches": n,
               "fetch_kib_raw": fk, "write_kib_raw": wk, "fetch_scale": fetch_scale, "write_scale": write_scale,
               "read_bytes_per_launch": fk * fetch_scale * 1024, "write_bytes_per_launch": wk * write_scale * 1024}
        rec["hbm_bytes_per_launch"] = rec["read_bytes_per_launch"] + rec["write_bytes_per_launch"]
        with open(os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"traffic_{rec_name}.json"), "w") as f:
            json.dump(rec, f, indent=1)
        log(f"{rec_name}: read {rec['read_bytes_per_launch'] / 1e6:.1f} MB, write "
            f"{rec['write_bytes_per_launch'] / 1e6:.1f} MB per launch ({n} dispatches); "
            f"scales {fetch_scale:.4f} / {write_scale:.4f}")


def measured_mfma_peak(A, torch):
    """Sustained bf16 MFMA rate of this device: the library's probe loop
    (independent accumulators, every CU busy), in TFLOP/s."""
    nb, iters = 2048, 200
    out = torch.empty(nb * 256, dtype=torch.float32, device="cuda")
    A.mfma_probe(out, nb, 10)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        A.mfma_probe(out, nb, iters)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, nb * iters * A.MFMA_PROBE_FLOP_PER_BLOCK_ITER / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return best


def unit_rates(A, torch):
    """Sustained rates of the units the attention kernels share, from the
    library's probe loops: LDS reads (TB/s and bytes per clock per CU at the
    nominal 2.4 GHz), fp32 FMA and exp2 issue rates (wave64 instructions per
    SIMD per nominal clock; the exp2 loop pairs each v_exp_f32 with one
    multiply)."""
    def best_ms(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        return best

    clk, cus, simds = 2.4e9, 256, 1024
    nb, it = 2048, 2000
    out = torch.empty(nb * 512, dtype=torch.float32, device="cuda")
    ms = best_ms(lambda: A.lds_probe(out, nb, it))
    lds = nb * 512 * 256 * it / (ms * 1e-3)
    rates = {"lds_read_TBps": lds / 1e12, "lds_read_B_per_clk_per_cu": lds / cus / clk}
    nb, it = 8192, 1000
    out = torch.empty(nb * 256, dtype=torch.float32, device="cuda")
    for name, e in (("fma", False), ("exp2_plus_mul", True)):
        ms = best_ms(lambda: A.valu_probe(out, nb, it, e))
        rates[f"{name}_wave64_per_simd_clk"] = nb * 4 * 16 * it / (ms * 1e-3) / simds / clk
    rates["exp2_cycles_est"] = 1 / rates["exp2_plus_mul_wave64_per_simd_clk"] - 1 / rates["fma_wave64_per_simd_clk"]
    return rates


def copy_bandwidth(torch):
    """Device-to-device copy rate (read + write bytes per second), GB/s."""
    src = torch.ones(1 << 27, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbps = 5 * 2 * src.numel() * 2 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return gbps


def skip_cost(A, torch, steps, warmup, copy_gbps):
    """The response-long workload (4 x 4352) and the same packs in rows
    padded to 8448 tokens: skipped tiles should cost nothing beyond writing
    the pad rows' zero outputs (predicted from the copy bandwidth)."""
    from workloads.generate import make_workload, pad_to_len
    w = make_workload(4, 0)
    ps = w.packset
    dev = torch.device("cuda:0")
    att = lambda p: p["fwd"] + p["bwd_dq"] + p["bwd_dkdv"]  # noqa: E731
    ts = {}
    for S_new in (ps.S, 8448):
        pps = pad_to_len(ps, S_new)
        t = []
        for x in (w.q, w.k, w.v, w.do):
            y = torch.zeros((x.shape[0], S_new) + tuple(x.shape[2:]), dtype=x.dtype)
            y[:, :ps.S] = x
            t.append(y.to(dev).contiguous())
        r = Runner(A, torch, pps, *t, w.Hq, w.Hkv, w.D, w.scale)
        _, per = time_runner(torch, r, steps, warmup)
        ts[S_new] = att(per)
        del r, t
    pad = ps.B * (8448 - ps.S)
    fill_bytes = pad * (2 * w.Hq * w.D * 2 + 2 * w.Hkv * w.D * 2 + w.Hq * 4)  # O, dQ, dK, dV, LSE of pad rows
    fill_ms = fill_bytes / (copy_gbps * 1e9 / 2) * 1e3  # writes at half the copy (read + write) rate
    extra_ms = ts[8448] - ts[ps.S] - fill_ms
    return {"workload": "response_long 4 x 4352 vs rows padded to 8448", "attn_ms": ts[ps.S], "attn_ms_padded": ts[8448],
            "pad_output_bytes": fill_bytes, "predicted_fill_ms": fill_ms, "excess_ms": extra_ms,
            "excess_frac": extra_ms / ts[ps.S]}


def delta_pass(A, torch, r, ps, w, n=20):
    """The row statistics of the backward ("LSE pass"): the forward writes
    LSE (4 bytes per valid row and q head); the dQ kernel's prologue reads O
    and dO (2 * 2 * D bytes per valid row and q head) and writes -Delta =
    -rowsum(dO * O) and -LSE / scale (8 bytes; the dK/dV kernel's
    accumulators start from them).  It is fused into that prologue, so it
    is timed as the dQ kernel on a copy of the map whose query tiles visit
    only their first key tile: the prologue (Q, dO, O loads, the two row
    stores), one tile, and the dQ block.  GB/s =
    algorithmic bytes of the pass / that time, a lower bound on the pass's
    own rate (the run also holds one tile's work, Q's loads and dQ's
    stores; all-pad tiles, which read nothing, are included as in the
    real kernel)."""
    m = A.BlockMap(ps.B, ps.S, *r.ftile)
    nb = A.map_bytes(ps.B, ps.S, *r.ftile)
    m.buffer[m._off0:m._off0 + nb].copy_(r.fmap.buffer[r.fmap._off0:r.fmap._off0 + nb])
    c = m.q2k_cnt()
    nfull = c[:, :, 0].clamp(max=1)
    c[:, :, 1] = torch.where(nfull > 0, torch.zeros_like(nfull), c[:, :, 1].clamp(max=1))
    c[:, :, 0] = nfull
    dq = torch.empty_like(r.dq)
    run = lambda: A.packed_attn_bwd(m, r.bmap, r.q, r.k, r.v, r.o, r.lse, r.do, r.scale,  # noqa: E731
                                    out=(dq, r.dk, r.dv), workspace=r.ws, stages=A.BWD_DQ)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    t_valid = ps.real_tokens()
    alg = (2 * 2 * w.D + 8) * w.Hq * t_valid          # O, dO read; -Delta, -LSE/scale written
    del m, dq
    return {"fwd_lse_write_bytes": 4 * w.Hq * t_valid, "algorithmic_bytes": alg, "prologue_one_tile_ms": ms,
            "GBps_lower_bound": alg / (ms * 1e-3) / 1e9, "frac_of_hbm_peak": alg / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "method": "dQ kernel with every visit list cut to its first key tile"}


def logp_rate(A, torch, r, pos_out, ps, V=151936):
    """Time pba_packed_token_logp on bf16 logits [B, S, V] (seeded normal,
    std 2.5) for the workload's response tokens: HBM bytes = one logits row
    (2 V bytes) per loss term, the rest is negligible."""
    g = torch.Generator(device="cuda").manual_seed(0)
    logits = (torch.randn((ps.B, ps.S, V), generator=g, device="cuda", dtype=torch.float32) * 2.5).to(torch.bfloat16)
    tokens = torch.randint(0, V, (ps.B, ps.S), generator=g, device="cuda", dtype=torch.int32)
    _, src, mask = pos_out
    tok = torch.empty((ps.B, ps.S), dtype=torch.float32, device="cuda")
    resp = torch.empty(r.R.numel(), dtype=torch.float32, device="cuda")
    for _ in range(2):
        A.packed_token_logp(r.fmap, src, mask, logits, tokens, r.P, r.R, out=(tok, resp))
    torch.cuda.synchronize()
    n = 10
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        A.packed_token_logp(r.fmap, src, mask, logits, tokens, r.P, r.R, out=(tok, resp))
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    terms = int(mask.sum())
    nbytes = terms * V * 2
    del logits
    return {"vocab": V, "loss_terms": terms, "ms": ms, "hbm_bytes": nbytes,
            "GBps": nbytes / (ms * 1e-3) / 1e9, "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}, resp


def cpu_baseline(w, seconds, gpu=None):
    """The fp64 oracle (dense masked attention + naive backward) on a bounded
    sample of the same workload: whole (batch row, kv group) units, in order,
    until `seconds` of wall time have been spent.  With `gpu` (the timed
    run's outputs on the host), its results on the same units are compared
    with the oracle's, outside the timed region."""
    import torch
    import oracle
    from workloads.generate import descriptor_arrays
    cores = len(os.sched_getaffinity(0))
    torch.set_num_threads(cores)
    ps = w.packset
    P, R = descriptor_arrays(ps)
    pk, br, _ = oracle.token_ids(P, R, ps.B, ps.S)
    G = w.Hq // w.Hkv
    flops, dense, units, t_used = 0.0, 0.0, [], 0.0
    err = {"o_max_abs": 0.0, "lse_max_abs": 0.0}
    sq = {x: [0.0, 0.0] for x in ("o", "dq", "dk", "dv")}  # squared error, squared reference
    for b in range(ps.B):
        mb = oracle.attention_mask(pk, br, row=b)
        n_allowed = int(mb.sum())
        valid = torch.from_numpy(pk[b] >= 0)
        for g in range(w.Hkv):
            t0 = time.perf_counter()
            rowmask = _RowMask(mb, b)
            hs = range(g * G, (g + 1) * G)
            O, L = oracle.attn_fwd(w.q, w.k, w.v, rowmask, w.scale, rows=[b], heads=hs)
            dq, dk, dv = oracle.attn_bwd(w.q, w.k, w.v, w.do, rowmask, w.scale, rows=[b], groups=[g])
            t_used += time.perf_counter() - t0
            if gpu is not None:
                h0, h1 = g * G, (g + 1) * G
                pairs = (("o", gpu["o"][b, :, h0:h1], O[b, :, h0:h1]), ("dq", gpu["dq"][b, :, h0:h1], dq[b, :, h0:h1]),
                         ("dk", gpu["dk"][b, :, g], dk[b, :, g]), ("dv", gpu["dv"][b, :, g], dv[b, :, g]))
                for name, x, ref in pairs:
                    x, ref = x[valid].double(), ref[valid]
                    sq[name][0] += float(((x - ref) ** 2).sum())
                    sq[name][1] += float((ref ** 2).sum())
                    if name == "o":
                        err["o_max_abs"] = max(err["o_max_abs"], float((x - ref).abs().max()))
                lg, lr = gpu["lse"][b, h0:h1][:, valid].double(), L[b, h0:h1][:, valid]
                err["lse_max_abs"] = max(err["lse_max_abs"], float((lg - lr).abs().max()))
            flops += 14.0 * w.D * G * n_allowed
            dense += 14.0 * w.D * G * float(ps.S) ** 2
            units.append((b, g))
            if t_used >= seconds:
                break
        if t_used >= seconds:
            break
    cpu = platform.processor() or platform.machine()
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    out = {"value": flops / t_used / 1e12, "unit": "TFLOP/s", "cores": torch.get_num_threads(), "kind": "oracle",
           "sample": f"{len(units)} of {ps.B * w.Hkv} (row, kv group) units, fp64 fwd+bwd, {t_used:.1f} s",
           "cpu_model": cpu, "wall_s": t_used, "units": len(units), "units_total": ps.B * w.Hkv,
           "dense_fp64_GFLOPs": dense / t_used / 1e9,
           "dense_work_note": "14*D*G*S^2 per (row, kv group) unit: the oracle computes the whole masked S x S square"}
    if gpu is not None:
        err.update({f"{x}_rel_l2": (sq[x][0] / sq[x][1]) ** 0.5 if sq[x][1] > 0 else 0.0 for x in sq})
        out["parity_on_sample"] = err
    return out


class _RowMask:
    """Indexable stand-in for a [B, S, S] mask that holds one row's mask."""

    def __init__(self, mb, b):
        self.mb, self.b = mb, b

    def __getitem__(self, i):
        assert i == self.b
        return self.mb


def config_sweep(A, torch, steps, warmup, cfgs=(3, 4, 5)):
    """The step on the larger workloads (context for the headline one): useful
    TFLOP/s per workload, each timed like the headline step."""
    from workloads.generate import make_workload
    dev = torch.device("cuda:0")
    out = {}
    for c in cfgs:
        w = make_workload(c, 0)
        t = [x.to(dev).contiguous() for x in (w.q, w.k, w.v, w.do)]
        r = Runner(A, torch, w.packset, *t, w.Hq, w.Hkv, w.D, w.scale)
        ms, per = time_runner(torch, r, steps, warmup)
        useful = 14.0 * w.D * w.Hq * allowed_pairs(w.packset)
        out[w.name] = {"B": w.packset.B, "S": w.packset.S, "ms_per_step": ms, "useful_tflops": useful / (ms * 1e-3) / 1e12,
                       "kernels_ms": {k_: round(v_, 4) for k_, v_ in per.items()}}
        del r, t
        torch.cuda.empty_cache()
    return out


def rope_rate(A, torch, r, q, k, base=1e6):
    """pba_packed_rope on the workload's Q (Hq heads) and K (Hkv heads), out
    of place: HBM bytes = read + write of each tensor."""
    yq, yk = torch.empty_like(q), torch.empty_like(k)
    for _ in range(2):
        A.packed_rope(r.fmap, q, base, out=yq)
        A.packed_rope(r.fmap, k, base, out=yk)
    torch.cuda.synchronize()
    n = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        A.packed_rope(r.fmap, q, base, out=yq)
        A.packed_rope(r.fmap, k, base, out=yk)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    nbytes = 2 * (q.numel() + k.numel()) * 2
    del yq, yk
    return {"ms_q_and_k": ms, "hbm_bytes": nbytes, "GBps": nbytes / (ms * 1e-3) / 1e9,
            "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}


def rope_step_cost(A, torch, r, q, k, v, do, scale, base=1e6, n=10):
    """The attention step with rotary inputs two ways: unfused (rotation
    passes on Q and K, plain forward and backward, inverse passes on dQ and
    dK) and fused (K pass, forward rotating Q in registers and writing the
    rotated Q, backward rotating dQ and dK back in its epilogues)."""
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    qr, kr = torch.empty_like(q), torch.empty_like(k)
    o, lse = torch.empty_like(q), torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32,
                                               device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def unfused():
        A.packed_rope(r.fmap, q, base, out=qr)
        A.packed_rope(r.fmap, k, base, out=kr)
        A.packed_attn_fwd(r.fmap, qr, kr, v, scale, out=(o, lse))
        A.packed_attn_bwd(r.fmap, r.bmap, qr, kr, v, o, lse, do, scale, out=(dq, dk, dv), workspace=r.ws)
        A.packed_rope(r.fmap, dq, base, inverse=True, out=dq)
        A.packed_rope(r.fmap, dk, base, inverse=True, out=dk)

    def fused():
        A.packed_rope(r.fmap, k, base, out=kr)
        A.packed_attn_fwd_rope(r.fmap, q, kr, v, base, scale, out=(o, lse), q_rot_out=qr)
        A.packed_attn_bwd_rope(r.fmap, r.bmap, qr, kr, v, o, lse, do, base, scale, out=(dq, dk, dv), workspace=r.ws)

    out = {}
    for name, fn in (("unfused_ms", unfused), ("fused_ms", fused)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name] = e0.elapsed_time(e1) / n
    out["base"] = base
    del qr, kr, o, lse, dq, dk, dv
    return out


def group_coef_time(A, torch, r, resp_logp):
    """pba_group_coefficients on the workload's packs (one group per pack,
    response 0 preferred), policy and reference sums from the log-prob run."""
    import numpy as np
    P = r.P.cpu().numpy().reshape(-1, 5)
    nresp = [int(x) for x in P[:, 3]]
    flags = []
    for k_ in nresp:
        flags += [1] + [0] * (k_ - 1)
    gp, mem, pos = (x.cuda() for x in A.groups_from_packs(nresp, flags))
    ref = resp_logp * 1.01
    for _ in range(3):
        out = A.group_coefficients(gp, mem, pos, resp_logp, ref, r.R, 0.1, "all_pairs")
    torch.cuda.synchronize()
    n = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        A.group_coefficients(gp, mem, pos, resp_logp, ref, r.R, 0.1, "all_pairs", out=out)
    e1.record()
    torch.cuda.synchronize()
    return {"groups": len(nresp), "responses": int(np.sum(nresp)), "ms": e0.elapsed_time(e1) / n}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="2", help="workload 1..5 or 3alt (default 2: Qwen3-8B-shaped packs)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-baselines", action="store_true", help="skip the dense-map and pairwise-layout runs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_*.json from two rocprofv3 counter_collection.csv files "
                         "(FETCH_SIZE run, WRITE_SIZE run) and exit; uses no GPU")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic, workload="qwen3_8b_packs (8 x 1828 tokens, 32/8 heads, D=128)")
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path (packs and kv-head groups "
              "shard with no exchange). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from workloads.generate import make_workload, pairwise_packset, pairwise_tensors
    import block_sparse_attention_pack_amd as pkg
    A = pkg.api

    cfg = parse_cfg(args.config)
    w = make_workload(cfg, 0)
    ps = w.packset
    dev = torch.device("cuda:0")
    q, k, v, do = (x.to(dev).contiguous() for x in (w.q, w.k, w.v, w.do))
    torch.cuda.synchronize()
    n_allowed = allowed_pairs(ps)
    useful = 14.0 * w.D * w.Hq * n_allowed
    log(f"workload {w.name}: B={ps.B} S={ps.S} Hq={w.Hq} Hkv={w.Hkv} D={w.D} allowed={n_allowed} "
        f"useful={useful:.3e} FLOP/step")

    r = Runner(A, torch, ps, q, k, v, do, w.Hq, w.Hkv, w.D, w.scale)
    ms, per = time_runner(torch, r, args.steps, args.warmup)
    tot = r.fmap.totals().cpu().tolist()
    totb = r.bmap.totals().cpu().tolist()
    value = useful / (ms * 1e-3) / 1e12
    log(f"step {ms:.3f} ms  useful {value:.1f} TFLOP/s  per-kernel ms {json.dumps({k_: round(v_, 4) for k_, v_ in per.items()})}")

    # Useful FLOPs per allowed (query, key) pair and q head: 4*D forward,
    # 10*D backward (Q K^T again, dO V^T, P^T dO, dS^T Q, dS K).  Each
    # backward kernel is credited only with work the other does not repeat:
    # P^T dO and dS^T Q (4*D) are the dK/dV kernel's alone, dS K (2*D) the
    # dQ kernel's alone, and Q K^T and dO V^T, which both form, count half
    # to each (2*D each): 6*D for dK/dV, 4*D for dQ, 10*D together.  The MFMA
    # work each kernel issues on allowed pairs (dK/dV 8*D, dQ 6*D, recomputed
    # products included) is reported beside it.
    credit = {"fwd": 4.0, "bwd_dq": 4.0, "bwd_dkdv": 6.0}
    issued = {"fwd": 4.0, "bwd_dq": 6.0, "bwd_dkdv": 8.0}
    rate = lambda f, t_ms: f * w.D * w.Hq * n_allowed / (t_ms * 1e-3) / 1e12  # noqa: E731
    kern = {name: {"ms": per[name], "useful_tflops_credited": rate(credit[name], per[name]),
                   "credited_flop_per_allowed_pair_per_head": credit[name] * w.D,
                   "mfma_tflops_issued_on_allowed_pairs": rate(issued[name], per[name]),
                   "issued_flop_per_allowed_pair_per_head": issued[name] * w.D}
            for name in credit}
    kern["map"] = {"ms": per["map"], "GBps": (map_bytes(r, r.fmap) + map_bytes(r, r.bmap)) / (per["map"] * 1e-3) / 1e9}
    dom = max(credit, key=lambda k_: per[k_])
    achieved = kern[dom]["useful_tflops_credited"]
    tr = traffic_record(dom)
    t_pair = per["bwd_dq"] + per["bwd_dkdv"]
    roofline = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": (tr["hbm_bytes_per_launch"] if tr else None),
                "credited_flop_per_allowed_pair_per_head": credit[dom] * w.D,
                "frac_issued": kern[dom]["mfma_tflops_issued_on_allowed_pairs"] / PEAK_BF16_TFLOPS,
                "frac_bwd_pair": rate(10.0, t_pair) / PEAK_BF16_TFLOPS,
                "frac_fwd": rate(4.0, per["fwd"]) / PEAK_BF16_TFLOPS}

    extra = {"skip_frac_fwd_tiles": tot[2] / max(1, sum(tot)), "tiles_fwd": {"full": tot[0], "partial": tot[1], "skip": tot[2],
             "shape": list(r.ftile)},
             "skip_frac_bwd_tiles": totb[2] / max(1, sum(totb)), "tiles_bwd": {"full": totb[0], "partial": totb[1],
             "skip": totb[2], "shape": list(r.btile)},
             "kernels": kern, "frac_of_peak": value / PEAK_BF16_TFLOPS, "allowed_pairs": n_allowed,
             "useful_flop_per_step": useful, "step_ms_events": per["step_events"],
             "useful_tflops_map_excluded": useful / ((per["fwd"] + per["bwd_dq"] + per["bwd_dkdv"]) * 1e-3) / 1e12}

    if not args.no_baselines:
        rd = Runner(A, torch, ps, q, k, v, do, w.Hq, w.Hkv, w.D, w.scale, dense=True)
        ms_d, per_d = time_runner(torch, rd, args.steps, args.warmup)
        att = lambda p: p["fwd"] + p["bwd_dq"] + p["bwd_dkdv"]  # noqa: E731
        del rd
        pps, pairs = pairwise_packset(ps)
        pt = [pairwise_tensors(x, pairs, pps.S).to(dev).contiguous() for x in (w.q, w.k, w.v, w.do)]
        rp = Runner(A, torch, pps, *pt, w.Hq, w.Hkv, w.D, w.scale)
        ms_p, per_p = time_runner(torch, rp, args.steps, args.warmup)
        del rp, pt
        extra.update({
            "attn_ms_sparse": att(per), "attn_ms_dense_map": att(per_d), "attn_ms_pairwise": att(per_p),
            "speedup_vs_dense_packed": att(per_d) / att(per),
            "speedup_vs_pairwise": att(per_p) / att(per),
            "pairwise_layout": {"B": pps.B, "S": pps.S, "allowed_pairs": allowed_pairs(pps)},
        })
        log(f"dense-map attn {att(per_d):.3f} ms, pairwise attn {att(per_p):.3f} ms, sparse attn {att(per):.3f} ms")

    if not args.no_baselines:
        # Context only: the same step once the device has run it for a
        # while.  A fresh process runs its first ~60 steps up to 15% slower
        # (other load beforehand does not remove this, only the step itself
        # does), so `value` above, taken after W warm-up steps, sits on that
        # ramp.
        t_ss = time.perf_counter()
        while time.perf_counter() - t_ss < 0.4:
            r.step()
            torch.cuda.synchronize()
        ms_ss, per_ss = time_runner(torch, r, args.steps, 0)
        extra["steady_state"] = {"after_seconds_of_steps": 0.4, "ms_per_step": ms_ss,
                                 "useful_tflops": useful / (ms_ss * 1e-3) / 1e12,
                                 "kernels_ms": {k_: round(v_, 4) for k_, v_ in per_ss.items()}}
        log(f"steady state: step {ms_ss:.3f} ms, useful {useful / (ms_ss * 1e-3) / 1e12:.1f} TFLOP/s")

    if not args.no_baselines:  # (profiled runs time only the step's own launches of each kernel)
        extra["lse_delta_pass"] = delta_pass(A, torch, r, ps, w)
        log(f"lse / delta pass: {json.dumps(extra['lse_delta_pass'])}")

    # Aligned positions / log-prob gather rows (a next step on the same map, reported beside the step).
    pos_out = (torch.empty((ps.B, ps.S), dtype=torch.int32, device=dev),
               torch.empty((ps.B, ps.S), dtype=torch.int32, device=dev),
               torch.empty((ps.B, ps.S), dtype=torch.uint8, device=dev))
    for _ in range(3):
        A.pack_positions(r.fmap, out=pos_out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        A.pack_positions(r.fmap, out=pos_out)
    e1.record()
    torch.cuda.synchronize()
    pos_ms = e0.elapsed_time(e1) / 20
    pos_bytes = ps.B * ps.S * (4 + 4 + 16 + 4 + 4 + 1)
    extra["positions"] = {"ms": pos_ms, "GBps": pos_bytes / (pos_ms * 1e-3) / 1e9, "bytes": pos_bytes}
    log(f"positions {pos_ms * 1e3:.1f} us")

    # Rotary embedding at the packed positions (a step before attention, reported beside the step).
    extra["rope"] = rope_rate(A, torch, r, q, k)
    if not args.no_baselines:
        extra["rope"]["attention_step"] = rope_step_cost(A, torch, r, q, k, v, do, w.scale)
    log(f"rope: {json.dumps(extra['rope'])}")

    # Packed token log-probs over a Qwen3-sized vocabulary (a next step after attention, reported beside the step).
    extra["logp"], resp_logp = logp_rate(A, torch, r, pos_out, ps)
    log(f"token log-probs: {json.dumps(extra['logp'])}")
    if (r.R > 0).all():
        extra["group_coef"] = group_coef_time(A, torch, r, resp_logp)
        log(f"group coefficients: {json.dumps(extra['group_coef'])}")

    peak_meas = measured_mfma_peak(A, torch)
    extra["measured_mfma_peak_tflops"] = peak_meas
    extra["frac_of_measured_peak"] = value / peak_meas
    roofline["frac_of_measured_peak"] = achieved / peak_meas
    log(f"measured MFMA peak {peak_meas:.0f} TFLOP/s: step at {value / peak_meas:.3f}, {dom} at {achieved / peak_meas:.3f}")
    extra["unit_rates"] = unit_rates(A, torch)
    log(f"unit rates: {json.dumps({k_: round(v_, 3) for k_, v_ in extra['unit_rates'].items()})}")
    if not args.no_baselines:
        gbps = copy_bandwidth(torch)
        extra["copy_GBps"] = gbps
        extra["skip_cost"] = skip_cost(A, torch, max(5, args.steps // 2), 2, gbps)
        log(f"skip cost: {json.dumps(extra['skip_cost'])}")

    if not args.no_baselines:
        extra["other_workloads"] = config_sweep(A, torch, max(5, args.steps // 2), 2)
        log(f"other workloads: {json.dumps({k_: round(v_['useful_tflops'], 1) for k_, v_ in extra['other_workloads'].items()})}")

    if args.copy_calibration:
        # 2^28 bytes read and 2^28 bytes written per launch, 3 launches.
        src = torch.ones(1 << 27, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host ...")
        gpu = {"o": r.o.cpu(), "lse": r.lse.cpu(), "dq": r.dq.cpu(), "dk": r.dk.cpu(), "dv": r.dv.cpu()}
        cpu = cpu_baseline(w, args.cpu_seconds, gpu)
        log(f"cpu baseline {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads; parity on that sample: "
            f"{json.dumps(cpu.get('parity_on_sample'))}")

    out = {
        "metric": "useful TFLOP/s packed-attention fwd+bwd (unmasked FLOPs); % bf16 MFMA peak",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded lognormal pack lengths standing in for UltraFeedback-style preference data)",
        "config": {"workload": w.name, "batch": ps.B, "seq_len": ps.S, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.D, "packs": len(ps.packs), "real_tokens": ps.real_tokens()},
        "roofline": roofline, "cpu_baseline": cpu, "extra": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
