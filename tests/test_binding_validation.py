"""The Python binding rejects mismatched tensors with ValueError before any
pointer reaches the library (a wrong shape, dtype or device would otherwise
become out-of-bounds device accesses), and outputs that overlap an input or
each other.  The CPU tests need no device (host tensors are refused before
anything touches one); the gpu-marked ones need device tensors but launch
no kernel."""
import pytest
import torch

import block_sparse_attention_pack_amd as P

A = P.api


def _bf(*shape, device="cpu"):
    return torch.zeros(shape, dtype=torch.bfloat16, device=device)


def test_host_tensors_are_refused():
    q, k = _bf(1, 8, 2, 64), _bf(1, 8, 2, 64)
    with pytest.raises(ValueError, match="device"):
        A.packed_attn_fwd(None, q, k, k)
    with pytest.raises(ValueError, match="device"):
        A.packed_attn_bwd(None, None, q, k, k, q, torch.zeros(1, 2, 8), q)
    with pytest.raises(ValueError, match="device"):
        A.packed_rope(None, q)
    with pytest.raises(ValueError, match="device"):
        A.packed_attn_fwd_rope(None, q, k, k, 1e4)
    with pytest.raises(ValueError, match="device"):
        A.pack_block_map(torch.zeros((1, 5), dtype=torch.int32), torch.zeros(1, dtype=torch.int32), 1, 8, 64, 64)


def test_wrong_dtypes_are_refused():
    with pytest.raises(ValueError, match="bfloat16"):
        A.packed_attn_fwd(None, torch.zeros(1, 8, 2, 64), _bf(1, 8, 2, 64), _bf(1, 8, 2, 64))
    with pytest.raises(ValueError, match="int32"):
        A.pack_block_map(torch.zeros((1, 5), dtype=torch.int64), torch.zeros(1, dtype=torch.int32), 1, 8, 64, 64)
    f = torch.zeros(3)
    with pytest.raises(ValueError, match="int32"):
        A.group_coefficients(f, f, f, f, f, f, 0.1)


@pytest.mark.gpu
def test_mismatched_device_tensors_are_refused():
    dev = "cuda"
    B, S, Hq, Hkv, D = 1, 100, 4, 2, 64
    m = A.BlockMap(B, S, *A.fwd_tile(Hq, Hkv, D))
    km = A.BlockMap(B, S, *A.bwd_tile(Hq, Hkv, D))
    q, k, v = _bf(B, S, Hq, D, device=dev), _bf(B, S, Hkv, D, device=dev), _bf(B, S, Hkv, D, device=dev)
    lse = torch.zeros((B, Hq, S), device=dev)
    cases = [
        lambda: A.packed_attn_fwd(m, q, _bf(B, S, Hkv, 32, device=dev), v),           # k head dim
        lambda: A.packed_attn_fwd(m, q, k, _bf(B, S, Hq, D, device=dev)),             # v heads
        lambda: A.packed_attn_fwd(m, q, k, v, out=(_bf(B, S, Hq, D - 8, device=dev), lse)),
        lambda: A.packed_attn_fwd(m, q, k, v, out=(q.clone(), lse[:, :, :-1])),       # lse shape
        lambda: A.packed_attn_fwd(m, q, k, v, out=(q.clone(), lse.double())),         # lse dtype
        lambda: A.packed_attn_fwd(m, q, k, v, out=(q.clone(), lse.cpu())),            # lse on the host
        lambda: A.packed_attn_fwd(m, q[:, :, :, ::2].contiguous(), k, v),             # q head dim != k's
        lambda: A.packed_attn_fwd(A.BlockMap(B, S + 1, *A.fwd_tile(Hq, Hkv, D)), q, k, v),  # map rows
        lambda: A.packed_attn_fwd(m, q.transpose(1, 2), k, v),                        # not contiguous
        lambda: A.packed_attn_bwd(m, km, q, k, v, _bf(B, S, Hq, 32, device=dev), lse, q),   # o shape
        lambda: A.packed_attn_bwd(m, km, q, k, v, q, lse, _bf(B, S - 1, Hq, D, device=dev)),  # dout shape
        lambda: A.packed_attn_bwd(m, km, q, k, v, q, lse.cpu(), q),                   # lse on the host
        lambda: A.packed_attn_bwd(m, km, q, k, v, q, lse, q, out=(q.clone(), q.clone(), v.clone())),  # dk shape
        lambda: A.packed_attn_bwd(m, km, q, k, v, q, lse, q,
                                  workspace=torch.empty(16, dtype=torch.uint8, device=dev)),  # workspace size
        lambda: A.packed_attn_bwd(m, km, q, k, v, q, lse, q,
                                  workspace=torch.empty(1 << 20, dtype=torch.uint8)),  # workspace on the host
        lambda: A.packed_attn_fwd_rope(m, q, k, v, 1e4, q_rot_out=_bf(B, S, Hq, 32, device=dev)),
        lambda: A.packed_rope(m, q, out=_bf(B, S, Hq, 32, device=dev)),
        lambda: A.pack_positions(m, out=(torch.zeros((B, S), dtype=torch.int64, device=dev), None, None)),
    ]
    for i, case in enumerate(cases):
        with pytest.raises(ValueError):
            case()
            pytest.fail(f"case {i} was accepted")
    # and the well-formed call is still accepted
    torch.cuda.synchronize()


def test_overlap_detection_on_host_buffers():
    """The overlap rule itself, on host memory (no device needed)."""
    from block_sparse_attention_pack_amd._lib import _disjoint
    buf = torch.zeros(1000, dtype=torch.uint8)
    a, b, c = buf[:400], buf[400:800], buf[399:401]
    _disjoint({"a": a}, {"b": b})                     # adjacent, disjoint
    _disjoint({"a": a, "b": b}, {})
    _disjoint({"e": buf[:0]}, {"a": a})               # empty tensors overlap nothing
    with pytest.raises(ValueError, match="a overlaps c"):
        _disjoint({"a": a}, {"c": c})
    with pytest.raises(ValueError, match="b overlaps c"):
        _disjoint({"b": b}, {"c": c})
    with pytest.raises(ValueError, match="a overlaps b"):
        _disjoint({"a": buf[:401], "b": b}, {})       # two outputs


@pytest.mark.gpu
def test_outputs_overlapping_inputs_are_refused():
    dev = "cuda"
    B, S, Hq, Hkv, D = 1, 100, 4, 2, 64
    m = A.BlockMap(B, S, *A.fwd_tile(Hq, Hkv, D))
    km = A.BlockMap(B, S, *A.bwd_tile(Hq, Hkv, D))
    q, k, v = _bf(B, S, Hq, D, device=dev), _bf(B, S, Hkv, D, device=dev), _bf(B, S, Hkv, D, device=dev)
    o, do = _bf(B, S, Hq, D, device=dev), _bf(B, S, Hq, D, device=dev)
    lse = torch.zeros((B, Hq, S), device=dev)
    need = A.workspace_bytes(B, S, Hq, D) + 256
    big = torch.zeros(need + q.numel() * 2, dtype=torch.uint8, device=dev)
    do_in_ws = big[need:].view(torch.bfloat16).view(q.shape)
    dkv = k.clone()
    cases = [
        lambda: A.packed_attn_fwd(m, q, k, v, out=(q, lse)),                                   # o is q
        lambda: A.packed_attn_fwd_rope(m, q, k, v, 1e4, q_rot_out=q),                          # q_rot is q
        lambda: A.packed_attn_bwd(m, km, q, k, v, o, lse, do, out=(q, k.clone(), v.clone())),  # dq is q
        lambda: A.packed_attn_bwd(m, km, q, k, v, o, lse, do, out=(do, k.clone(), v.clone())),  # dq is dout
        lambda: A.packed_attn_bwd(m, km, q, k, v, o, lse, do, out=(q.clone(), dkv, dkv)),        # dk is dv
        lambda: A.packed_attn_bwd(m, km, q, k, v, o, lse, do_in_ws, workspace=big),            # workspace holds dout
        lambda: A.packed_attn_bwd_noalloc(m, km, q, k, v, o, lse, do, out=(o, k.clone(), v.clone())),
    ]
    for i, case in enumerate(cases):
        with pytest.raises(ValueError, match="overlaps"):
            case()
            pytest.fail(f"case {i} was accepted")
    torch.cuda.synchronize()
