"""The C-ABI library loads, exports every declared symbol, and rejects bad
host arguments synchronously (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "block_sparse_attention_pack_amd", "libpba.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from block_sparse_attention_pack_amd.build import build
        build()
    return ctypes.CDLL(LIB)


def _declared(headers=None):
    """Every pba_* function declared in include/*.h (or the named headers)."""
    inc = os.path.join(ROOT, "include")
    names = set()
    for h in headers or sorted(f for f in os.listdir(inc) if f.endswith(".h")):
        src = open(os.path.join(inc, h)).read()
        names |= set(re.findall(r"PBA_API\s+[\w\s\*]+?\b(pba_\w+)\s*\(", src))
    return sorted(names)


def test_probes_live_outside_the_method_header():
    assert not {"pba_mfma_probe", "pba_lds_probe", "pba_valu_probe"} & set(_declared(["pba.h"]))
    assert {"pba_mfma_probe", "pba_lds_probe", "pba_valu_probe"} <= set(_declared(["pba_measure.h"]))


def test_header_declares_the_three_calls():
    names = _declared()
    for n in ("pba_pack_block_map", "pba_packed_attn_fwd", "pba_packed_attn_bwd"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in _declared():
        assert hasattr(lib, n), n


def test_binding_loads_and_lists_exports():
    import block_sparse_attention_pack_amd as P
    assert set(P.api.EXPORTED) == set(_declared())


def test_host_argument_errors():
    import block_sparse_attention_pack_amd as P
    A = P.api
    with pytest.raises(A.PbaError) as e:
        A.fwd_tile(32, 7, 128)
    assert e.value.code == -3
    with pytest.raises(A.PbaError) as e:
        A.fwd_tile(32, 8, 96)
    assert e.value.code == -4
    assert A.map_bytes(0, 10, 64, 64) == 0
    assert A.map_bytes(1, 10, 48, 64) == 0
    assert A.workspace_bytes(1, 10, 4, 80) == 0
    assert A.fwd_tile(32, 8, 128) == (32, 64)
    assert A.fwd_tile(4, 2, 64) == (64, 64)
    assert A.fwd_tile(2, 2, 64) == (128, 64)
    assert A.bwd_tile(32, 8, 128) == (64, 128)
    lib = A._lib
    # null map / null pointers are rejected before any device work
    assert lib.pba_pack_block_map(None, 0, None, 0, None, None) == -1
    assert lib.pba_packed_attn_fwd(None, 16, 16, 16, 16, 16, 1, 8, 2, 2, 64, 0.1, None) == -1
    m = A.PbaBlockMap()
    assert lib.pba_map_init(ctypes.byref(m), 256, 1 << 20, 2, 100, 64, 64) == 0
    assert (m.nqt, m.nkt) == (2, 2)
    assert lib.pba_map_init(ctypes.byref(m), 256 + 16, 1 << 20, 2, 100, 64, 64) == -9
    assert lib.pba_map_init(ctypes.byref(m), 256, 16, 2, 100, 64, 64) == -6
    # map shape mismatches are caught on the host
    assert lib.pba_packed_attn_fwd(ctypes.byref(m), 16, 16, 16, 16, 16, 2, 101, 4, 2, 64, 0.1, None) == -6
    assert lib.pba_packed_attn_fwd(ctypes.byref(m), 16, 16, 16, 16, 16, 2, 100, 4, 4, 64, 0.1, None) == -5
    assert lib.pba_packed_attn_fwd(ctypes.byref(m), 16, 16, 16, 16, 16, 2, 100, 4, 3, 64, 0.1, None) == -3
    assert lib.pba_packed_attn_fwd(ctypes.byref(m), 8, 16, 16, 16, 16, 2, 100, 4, 2, 64, 0.1, None) == -9
    ws = A.workspace_bytes(2, 100, 4, 64)
    assert ws >= 2 * 2 * 4 * 100 * 4
    mb = A.PbaBlockMap()
    assert lib.pba_map_init(ctypes.byref(mb), 256, 1 << 20, 2, 100, 64, 128) == 0
    # (4, 2, 64): forward / dQ tiles 64x64 (map m), dK / dV tiles 64x128 (map mb)
    args = [ctypes.byref(m), ctypes.byref(mb)] + [16] * 9
    assert lib.pba_packed_attn_bwd(*args, 256, 0, 2, 100, 4, 2, 64, 0.1, None) == -7
    assert lib.pba_packed_attn_bwd(*args, 256, ws - 1, 2, 100, 4, 2, 64, 0.1, None) == -7
    swapped = [ctypes.byref(mb), ctypes.byref(m)] + [16] * 9
    assert lib.pba_packed_attn_bwd(*swapped, 256, ws, 2, 100, 4, 2, 64, 0.1, None) == -5
    # the softmax scale must be positive and finite
    assert lib.pba_packed_attn_fwd(ctypes.byref(m), 16, 16, 16, 16, 16, 2, 100, 4, 2, 64, 0.0, None) == -10
    assert lib.pba_packed_attn_fwd(ctypes.byref(m), 16, 16, 16, 16, 16, 2, 100, 4, 2, 64, -0.1, None) == -10
    assert lib.pba_packed_attn_bwd(*args, 256, ws, 2, 100, 4, 2, 64, float("inf"), None) == -10
    # one batch row of Q must stay under 2 GiB (32-bit buffer offsets)
    assert lib.pba_packed_attn_fwd(ctypes.byref(m), 16, 16, 16, 16, 16, 2, 1 << 20, 16, 8, 128, 0.1, None) == -2


def test_positions_and_probe_argument_errors():
    import block_sparse_attention_pack_amd as P
    A = P.api
    lib = A._lib
    assert lib.pba_pack_positions(None, 16, 16, 16, None) == -1
    m = A.PbaBlockMap()
    assert lib.pba_map_init(ctypes.byref(m), 256, 1 << 20, 2, 100, 64, 64) == 0
    # nothing requested: nothing to do, no device needed
    assert lib.pba_pack_positions(ctypes.byref(m), None, None, None, None) == 0
    bad = A.PbaBlockMap()
    assert lib.pba_pack_positions(ctypes.byref(bad), 16, None, None, None) == -1
    assert lib.pba_mfma_probe(None, 1, 1, None) == -1
    assert lib.pba_mfma_probe(16, 0, 1, None) == -2
    assert lib.pba_mfma_probe(16, 1, 0, None) == -2
    assert lib.pba_lds_probe(None, 1, 1, None) == -1
    assert lib.pba_lds_probe(16, 0, 1, None) == -2
    assert lib.pba_valu_probe(None, 1, 1, 0, None) == -1
    assert lib.pba_valu_probe(16, 1, 0, 1, None) == -2
    assert lib.pba_valu_probe(16, 1, 1, 2, None) == -2


def test_group_coefficients_argument_errors():
    import block_sparse_attention_pack_amd as P
    lib = P.api._lib
    f = lib.pba_group_coefficients
    p = 16  # a non-NULL stand-in: every case below fails before any device access
    ok = dict(gp=p, G=1, mem=p, pos=p, E=2, pol=p, ref=p, rl=p, n=2, obj=0, beta=0.1, alpha=1.0, coef=p, nll=None,
              loss=None, st=p)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["gp"], a["G"], a["mem"], a["pos"], a["E"], a["pol"], a["ref"], a["rl"], a["n"], a["obj"], a["beta"],
                 a["alpha"], a["coef"], a["nll"], a["loss"], a["st"], None)

    for k in ("gp", "mem", "pos", "pol", "ref", "rl", "coef", "st"):
        assert call(**{k: None}) == -1, k
    assert call(E=1) == -2
    assert call(E=4097, G=2) == -2
    assert call(G=0) == -2
    assert call(G=2, E=3) == -2       # a group needs two entries
    assert call(n=0) == -2
    assert call(obj=4) == -11
    assert call(obj=-1) == -11
    assert call(beta=0.0) == -11
    assert call(beta=float("inf")) == -11
    assert call(alpha=-1.0) == -11
    assert call(alpha=float("nan")) == -11
    assert "group" in P.api.strerror(15) and "objective" in P.api.strerror(-11)


def test_rope_argument_errors():
    import block_sparse_attention_pack_amd as P
    A = P.api
    lib = A._lib
    m = A.PbaBlockMap()
    assert lib.pba_map_init(ctypes.byref(m), 256, 1 << 20, 2, 100, 64, 64) == 0
    assert lib.pba_packed_rope(None, 16, 16, 2, 64, 1e4, 0, None) == -1
    assert lib.pba_packed_rope(ctypes.byref(m), None, 16, 2, 64, 1e4, 0, None) == -1
    assert lib.pba_packed_rope(ctypes.byref(m), 16, 16, 0, 64, 1e4, 0, None) == -2
    assert lib.pba_packed_rope(ctypes.byref(m), 16, 16, 2, 96, 1e4, 0, None) == -4
    assert lib.pba_packed_rope(ctypes.byref(m), 16, 16, 2, 64, 1.0, 0, None) == -11
    assert lib.pba_packed_rope(ctypes.byref(m), 16, 16, 2, 64, float("inf"), 0, None) == -11
    assert lib.pba_packed_rope(ctypes.byref(m), 24, 16, 2, 64, 1e4, 0, None) == -9


def test_backward_workspace_layout():
    """Two fp32 [B, Hq, S] arrays, then the split area of the dK / dV stage:
    arrival counters (+1 for the split count) and 2 x 2 fp32 blocks of
    128 keys x D per (key tile, kv head) pair, at most 256 pairs."""
    import block_sparse_attention_pack_amd as P
    A = P.api
    al = lambda n: (n + 255) // 256 * 256  # noqa: E731
    for B, S, Hq, D in [(1, 144, 2, 64), (8, 1828, 32, 128), (2, 100, 4, 64), (1, 131072, 32, 128)]:
        pairs = min(256, B * -(-S // 128) * Hq)
        want = 2 * al(B * Hq * S * 4) + al((pairs + 1) * 4) + pairs * 2 * 2 * 128 * D * 4
        assert A.workspace_bytes(B, S, Hq, D) == want, (B, S, Hq, D)


def test_traffic_records_from_counter_csv(tmp_path):
    """bench.py --write-traffic: per-kernel averages of FETCH_SIZE / WRITE_SIZE,
    scaled by the 2^28-byte calibration copy (small copies ignored)."""
    import csv
    import json
    import bench

    names = {"fwd": "void pba::(anonymous namespace)::fwd_kernel<128, 4, false>(pba::FwdArgs)",
             "bwd_dq": "void pba::(anonymous namespace)::bwd_dq<128, 4>(pba::BwdArgs)",
             "bwd_dkdv": "void pba::(anonymous namespace)::bwd_dkdv<128>(pba::BwdArgs)"}

    def write(path, counter, copy_kib, vals):
        with open(path, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
            w.writeheader()
            w.writerow({"Kernel_Name": "__amd_rocclr_copyBuffer", "Grid_Size": 512, "Counter_Name": counter,
                        "Counter_Value": 3})
            for _ in range(3):
                w.writerow({"Kernel_Name": "__amd_rocclr_copyBuffer", "Grid_Size": 131072, "Counter_Name": counter,
                            "Counter_Value": copy_kib})
            for k, (a, b) in vals.items():
                for v in (a, b):
                    w.writerow({"Kernel_Name": names[k], "Grid_Size": 1024, "Counter_Name": counter,
                                "Counter_Value": v})

    write(tmp_path / "f.csv", "FETCH_SIZE", 131072, {"fwd": (100, 300), "bwd_dq": (10, 10), "bwd_dkdv": (1, 3)})
    write(tmp_path / "w.csv", "WRITE_SIZE", 262144, {"fwd": (50, 50), "bwd_dq": (20, 20), "bwd_dkdv": (2, 2)})
    bench.write_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "test", out_dir=str(tmp_path))
    rec = json.load(open(tmp_path / "traffic_fwd.json"))
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["read_bytes_per_launch"] == 200 * 2.0 * 1024
    assert rec["write_bytes_per_launch"] == 50 * 1024
    assert rec["sources_sha256"] == bench.sources_sha256(rec["sources"])
    assert json.load(open(tmp_path / "traffic_bwd_dkdv.json"))["read_bytes_per_launch"] == 2 * 2.0 * 1024


def test_noalloc_backward_argument_errors():
    """pba_packed_attn_bwd_noalloc checks its arguments as the workspace
    entry point does, and refuses a problem whose row statistics do not fit
    its fixed scratch, all before any device work."""
    import block_sparse_attention_pack_amd as P
    A = P.api
    lib = A._lib
    m, mb = A.PbaBlockMap(), A.PbaBlockMap()
    assert lib.pba_map_init(ctypes.byref(m), 256, 1 << 20, 2, 100, 64, 64) == 0
    assert lib.pba_map_init(ctypes.byref(mb), 256, 1 << 20, 2, 100, 64, 128) == 0
    args = [ctypes.byref(m), ctypes.byref(mb)] + [16] * 9
    assert lib.pba_packed_attn_bwd_noalloc(*([ctypes.byref(m), ctypes.byref(mb)] + [16] * 8 + [None]),
                                           2, 100, 4, 2, 64, 0.1, None) == -1
    assert lib.pba_packed_attn_bwd_noalloc(*args, 2, 101, 4, 2, 64, 0.1, None) == -6
    assert lib.pba_packed_attn_bwd_noalloc(*args, 2, 100, 4, 4, 64, 0.1, None) == -5
    assert lib.pba_packed_attn_bwd_noalloc(*args, 2, 100, 4, 2, 64, 0.0, None) == -10
    assert lib.pba_packed_attn_bwd_noalloc(*args, 2, 100, 4, 2, 96, 0.1, None) == -4
    # 16 rows of 32768 tokens x 32 q heads: 8 * B * Hq * S = 128 MiB of row
    # statistics against the 96 MiB scratch
    B, S = 16, 32768
    big_q, big_k = A.PbaBlockMap(), A.PbaBlockMap()
    assert lib.pba_map_init(ctypes.byref(big_q), 256, 1 << 40, B, S, *A.fwd_tile(32, 8, 128)) == 0
    assert lib.pba_map_init(ctypes.byref(big_k), 256, 1 << 40, B, S, *A.bwd_tile(32, 8, 128)) == 0
    big = [ctypes.byref(big_q), ctypes.byref(big_k)] + [16] * 9
    assert 8 * B * 32 * S > A.NOALLOC_SCRATCH_BYTES
    assert lib.pba_packed_attn_bwd_noalloc(*big, B, S, 32, 8, 128, 0.1, None) == -12
    assert "scratch" in A.strerror(-12)
