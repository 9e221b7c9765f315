"""GPU aligned positions / log-prob gather rows vs the oracle: bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from gpu_path import api, build_map, say
from oracle_pins import descriptors
from workloads.generate import Pack, PackSet, descriptor_arrays, make_packset, random_packset

pytestmark = pytest.mark.gpu


def _compare(ps, tile=(64, 64)):
    P, R = descriptor_arrays(ps)
    want = oracle.positions(P, R, ps.B, ps.S)
    m = build_map(ps, *tile)
    got = api().pack_positions(m)
    for g, w_, name in zip(got, want[:3], ("pos_ids", "src_row", "loss_mask")):
        np.testing.assert_array_equal(g.cpu().numpy(), w_, err_msg=f"{name} B={ps.B} S={ps.S}")


def test_tiny_config():
    say("positions tiny")
    _compare(make_packset(1))


@pytest.mark.parametrize("cfg", [2, 3, 4, 5, "3alt"])
def test_full_configs(cfg):
    ps = make_packset(cfg)
    say("positions config", cfg, ps.B, ps.S)
    _compare(ps, (128, 128))


@pytest.mark.parametrize("seed", range(8))
def test_random_ragged(seed):
    rng = np.random.default_rng(2000 + seed)
    ps = random_packset(rng, B=int(rng.integers(1, 4)), S=int(rng.integers(1, 700)), max_packs_per_row=5,
                        max_resp=6, max_len=int(rng.integers(2, 200)))
    say("positions random", seed, ps.B, ps.S, len(ps.packs))
    _compare(ps, [(64, 64), (32, 64), (16, 16)][seed % 3])


def test_edge_cases():
    cases = [
        PackSet(1, 1, [Pack(0, 0, 1, ())]),
        PackSet(1, 5, []),                                        # all pad
        PackSet(2, 70, [Pack(1, 0, 0, (0, 0, 70))]),              # empty prompt and empty branches
        PackSet(1, 130, [Pack(0, 0, 64, (0, 66))]),               # empty first response
        PackSet(1, 200, [Pack(0, 3, 5, ()), Pack(0, 8, 0, ()), Pack(0, 8, 0, (1,) * 40)]),
    ]
    for i, ps in enumerate(cases):
        say("positions edge", i)
        _compare(ps)


def test_null_outputs_and_invalid_map():
    A = api()
    ps = make_packset(1)
    m = build_map(ps, 64, 64)
    pos, src, mask = A.pack_positions(m)
    only = torch.full((ps.B, ps.S), 7, dtype=torch.int32, device="cuda")
    A.pack_positions(m, out=(None, only, None))
    assert torch.equal(only, src)
    # invalid descriptors: the map's status is set and nothing is written
    P, R = descriptors([(0, 0, 4, (3,)), (0, 2, 1, ())])
    pd, rd = A.descriptors_to_device(P, R)
    bad = A.pack_block_map(pd, rd, 1, 16, 64, 64)
    assert int(bad.status().cpu()[0]) != 0
    sentinel = [torch.full((1, 16), -5, dtype=torch.int32, device="cuda"),
                torch.full((1, 16), -5, dtype=torch.int32, device="cuda"),
                torch.full((1, 16), 9, dtype=torch.uint8, device="cuda")]
    A.pack_positions(bad, out=tuple(sentinel))
    torch.cuda.synchronize()
    assert (sentinel[0] == -5).all() and (sentinel[1] == -5).all() and (sentinel[2] == 9).all()
