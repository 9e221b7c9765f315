"""GPU block map vs the oracle's brute-force map: bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from gpu_path import api, build_map, say
from oracle_pins import descriptors
from workloads.generate import Pack, PackSet, descriptor_arrays, make_packset, random_packset

pytestmark = pytest.mark.gpu

FIELDS = ("tok_pack", "tok_branch", "tok_win", "cls", "q2k_cnt", "q2k_idx", "k2q_cnt", "k2q_idx", "totals", "status",
          "q_order", "k_order")


def _compare(ps, bm, bn):
    P, R = descriptor_arrays(ps)
    want = oracle.block_map(P, R, ps.B, ps.S, bm, bn)
    got = build_map(ps, bm, bn).to_host()
    for f in FIELDS:
        np.testing.assert_array_equal(got[f], want[f], err_msg=f"{f} B={ps.B} S={ps.S} tile={bm}x{bn}")


TILES = [(64, 64), (64, 128), (128, 64), (128, 128), (256, 64), (16, 32)]


@pytest.mark.parametrize("tile", TILES)
def test_tiny_config(tile):
    say("map tiny", tile)
    _compare(make_packset(1), *tile)


@pytest.mark.parametrize("seed", range(16))
def test_random_ragged(seed):
    rng = np.random.default_rng(1000 + seed)
    ps = random_packset(rng, B=int(rng.integers(1, 4)), S=int(rng.integers(1, 700)), max_packs_per_row=5,
                        max_resp=6, max_len=int(rng.integers(2, 200)))
    tile = TILES[seed % len(TILES)]
    say("map random", seed, ps.B, ps.S, len(ps.packs), tile)
    _compare(ps, *tile)


def test_edge_cases():
    cases = [
        PackSet(1, 1, [Pack(0, 0, 1, ())]),
        PackSet(1, 5, []),                                        # all pad
        PackSet(2, 70, [Pack(1, 0, 0, (0, 0, 70))]),              # zero-length branches, row 0 all pad
        PackSet(1, 130, [Pack(0, 0, 64, (0, 66))]),               # empty first response: one run
        PackSet(1, 200, [Pack(0, 3, 5, ()), Pack(0, 8, 0, ()), Pack(0, 8, 0, (1,) * 40)]),  # many tiny responses
    ]
    for i, ps in enumerate(cases):
        for tile in [(64, 64), (64, 128), (16, 16)]:
            say("map edge", i, tile)
            _compare(ps, *tile)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5, "3alt"])
def test_full_configs(cfg):
    ps = make_packset(cfg)
    A = api()
    for tile in {A.fwd_tile(32, 8, 128), A.bwd_tile(32, 8, 128), (128, 128)}:
        say("map config", cfg, tile)
        _compare(ps, *tile)


def test_descriptor_errors_set_status():
    S = oracle.STATUS
    cases = {
        "row": [(0, 0, 2, ()), (2, 0, 1, ())],
        "negative": [(0, 0, -1, ())],
        "bounds": [(0, 0, 5, (6,))],
        "order": [(0, 4, 2, ()), (0, 5, 1, ())],
    }
    A = api()
    for name, pl in cases.items():
        P, R = descriptors(pl)
        pd, rd = A.descriptors_to_device(P, R)
        say("map status", name)
        m = A.pack_block_map(pd, rd, 2, 10, 16, 16)
        torch.cuda.synchronize()
        want = oracle.token_ids(P, R, 2, 10)[2]
        assert tuple(m.status().cpu().tolist()) == tuple(want) and want[0] == S[name]
    P, R = descriptors([(0, 0, 2, (1,))])
    P[0, 4] = 5
    pd, rd = A.descriptors_to_device(P, R)
    m = A.pack_block_map(pd, rd, 2, 10, 16, 16)
    assert tuple(m.status().cpu().tolist()) == (S["resp_range"], 0)


def test_map_is_deterministic():
    ps = make_packset(3)
    a = build_map(ps, 64, 64).to_host()
    b = build_map(ps, 64, 64).to_host()
    for f in FIELDS:
        np.testing.assert_array_equal(a[f], b[f])


def _compare_multi(ps, tiles):
    """pba_pack_block_maps builds every map bit-exactly as the oracle does."""
    A = api()
    P, R = descriptor_arrays(ps)
    pd, rd = A.descriptors_to_device(P, R)
    maps = [A.BlockMap(ps.B, ps.S, bm, bn) for bm, bn in tiles]
    A.pack_block_maps(pd, rd, maps)
    for (bm, bn), m in zip(tiles, maps):
        want = oracle.block_map(P, R, ps.B, ps.S, bm, bn)
        got = m.to_host()
        for f in FIELDS:
            np.testing.assert_array_equal(got[f], want[f], err_msg=f"{f} B={ps.B} S={ps.S} tile={bm}x{bn}")


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_multi_map_build_configs(cfg):
    ps = make_packset(cfg)
    A = api()
    Hq, Hkv, D = (2, 2, 64) if cfg == 1 else (32, 8, 128)
    tiles = [A.fwd_tile(Hq, Hkv, D), A.bwd_tile(Hq, Hkv, D), (16, 32), (128, 128)]
    say("multi map", cfg, tiles)
    _compare_multi(ps, tiles)


@pytest.mark.parametrize("seed", range(4))
def test_multi_map_build_random(seed):
    rng = np.random.default_rng(3000 + seed)
    ps = random_packset(rng, B=int(rng.integers(1, 4)), S=int(rng.integers(1, 500)), max_packs_per_row=4,
                        max_resp=5, max_len=int(rng.integers(2, 150)))
    say("multi map random", seed, ps.B, ps.S, len(ps.packs))
    _compare_multi(ps, [(32, 64), (64, 128)])


def test_work_order_large_map():
    """More tiles per side than the order kernel sorts in LDS (2048): the
    chunked counting-sort path, still bit-exact."""
    rng = np.random.default_rng(77)
    ps = random_packset(rng, B=40, S=1000, max_packs_per_row=4, max_resp=4, max_len=120)
    say("map large order", ps.B, ps.S, len(ps.packs))
    _compare_multi(ps, [(16, 16), (16, 64)])


@pytest.mark.parametrize("S", [1024, 1025])
def test_work_order_at_the_lds_sort_limit(S):
    """Exactly 2048 tiles per side (sorted by rank in LDS by the last list
    workgroup) and 2080 (the counting-sort pass): both bit-exact."""
    rng = np.random.default_rng(91)
    ps = random_packset(rng, B=32, S=S, max_packs_per_row=3, max_resp=4, max_len=200)
    say("map order limit", ps.B, ps.S, len(ps.packs))
    _compare_multi(ps, [(16, 16), (16, 64)])
