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


def _declared():
    src = open(os.path.join(ROOT, "include", "pba.h")).read()
    return sorted(set(re.findall(r"PBA_API\s+[\w\s\*]+?\b(pba_\w+)\s*\(", src)))


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
