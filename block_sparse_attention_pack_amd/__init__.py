"""Packed branch-aware attention for MI355X (gfx950).

Attention over packed preference sequences [prompt | response_0 | ...]:
each response attends to the shared prompt and its own earlier tokens, never
to a sibling, several packs may share a row, and tiles the mask empties are
skipped.  The compute runs in libpba.so (hand-written HIP kernels); this
package is a thin ctypes binding (see include/pba.h for the C ABI).

    from block_sparse_attention_pack_amd import api
    fmap = api.pack_block_map(packs, resp_len, B, S, *api.fwd_tile(Hq, Hkv, D))
    o, lse = api.packed_attn_fwd(fmap, q, k, v)
    bmap = api.pack_block_map(packs, resp_len, B, S, *api.bwd_tile(Hq, Hkv, D))
    dq, dk, dv = api.packed_attn_bwd(bmap, q, k, v, o, lse, do)
"""


def __getattr__(name):
    # Load the library lazily so that building it does not need it.
    if name == "api":
        from . import _lib
        return _lib
    raise AttributeError(name)
