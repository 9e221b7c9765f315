"""Pins of the oracle's block map and per-token windows (CPU only)."""
import numpy as np
import pytest

import oracle
from oracle_pins import descriptors, pairwise_union_mask
from workloads.generate import descriptor_arrays, make_packset, random_packset


def _parse_map_fixture(path):
    lines = [l.rstrip("\n") for l in open(path) if l.strip() and not l.startswith("#")]
    out, i = {}, 0
    while i < len(lines):
        _, bm, bn = lines[i].split()
        key = (int(bm), int(bn))
        i += 1
        grid = []
        while lines[i] not in ("q2k",):
            grid.append([int(x) for x in lines[i].split()])
            i += 1
        i += 1
        lists = {"q2k": [], "k2q": []}
        cur = "q2k"
        while i < len(lines) and not lines[i].startswith("cls"):
            if lines[i] == "k2q":
                cur = "k2q"
            elif lines[i].startswith(("qorder:", "korder:")):
                name, rest = lines[i].split(":")
                lists[name] = [int(x) for x in rest.split()]
            else:
                _, rest = lines[i].split(":")
                full, part = rest.split("|")
                lists[cur].append(([int(x) for x in full.split()], [int(x) for x in part.split()]))
            i += 1
        out[key] = (np.array(grid, dtype=np.uint8), lists)
    return out


def test_tiny_pack_worked_map(golden_dir):
    fx = _parse_map_fixture(f"{golden_dir}/p1_tiny_pack_map.txt")
    P, R = descriptor_arrays(make_packset(1))
    for (bm, bn), (grid, lists) in fx.items():
        m = oracle.block_map(P, R, 1, 144, bm, bn)
        np.testing.assert_array_equal(m["cls"][0], grid)
        for name, cnt, idx in (("q2k", "q2k_cnt", "q2k_idx"), ("k2q", "k2q_cnt", "k2q_idx")):
            for t, (full, part) in enumerate(lists[name]):
                assert m[cnt][0, t].tolist() == [len(full), len(part)]
                n = len(full) + len(part)
                assert m[idx][0, t, :n].tolist() == full + part
                assert (m[idx][0, t, n:] == -1).all()
        assert m["q_order"].tolist() == lists["qorder"]
        assert m["k_order"].tolist() == lists["korder"]
    m = oracle.block_map(P, R, 1, 144, 64, 64)
    assert m["totals"].tolist() == [1, 5, 3]


def test_work_order_ties_across_rows():
    """Two identical rows of the tiny pack: visit counts per flat query tile
    are [1, 2, 3, 1, 2, 3], so longest-first with index tie-breaks gives
    [2, 5, 1, 4, 0, 3]; key tiles [3, 2, 1, 3, 2, 1] give [0, 3, 1, 4, 2, 5]."""
    P, R = descriptors([(0, 0, 64, (32, 48)), (1, 0, 64, (32, 48))])
    m = oracle.block_map(P, R, 2, 144, 64, 64)
    assert m["q_order"].tolist() == [2, 5, 1, 4, 0, 3]
    assert m["k_order"].tolist() == [0, 3, 1, 4, 2, 5]


@pytest.mark.parametrize("seed", range(6))
def test_work_order_is_a_sorted_permutation(seed):
    rng = np.random.default_rng(300 + seed)
    ps = random_packset(rng, B=3, S=int(rng.integers(30, 300)), max_packs_per_row=3, max_resp=4, max_len=60)
    P, R = descriptor_arrays(ps)
    m = oracle.block_map(P, R, ps.B, ps.S, 32, 16)
    for order, cnt in ((m["q_order"], m["q2k_cnt"]), (m["k_order"], m["k2q_cnt"])):
        visits = cnt.reshape(-1, 2).sum(axis=1)
        assert sorted(order.tolist()) == list(range(len(visits)))
        for a, b in zip(order[:-1], order[1:]):
            assert visits[a] > visits[b] or (visits[a] == visits[b] and a < b)


def _brute_cls(mask_b, S, BM, BN):
    nqt, nkt = -(-S // BM), -(-S // BN)
    cls = np.zeros((nqt, nkt), dtype=np.uint8)
    for qt in range(nqt):
        for kt in range(nkt):
            c = 0
            for i in range(qt * BM, qt * BM + BM):
                for j in range(kt * BN, kt * BN + BN):
                    if i < S and j < S and mask_b[i, j]:
                        c += 1
            cls[qt, kt] = 2 if c == BM * BN else (0 if c == 0 else 1)
    return cls


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("tile", [(4, 4), (8, 4), (4, 8), (8, 8)])
def test_map_against_loop_count_on_union_mask(seed, tile):
    rng = np.random.default_rng(100 + seed)
    ps = random_packset(rng, B=2, S=int(rng.integers(1, 40)), max_len=8)
    pl = [(p.row, p.start, p.prompt_len, p.resp_lens) for p in ps.packs]
    P, R = descriptor_arrays(ps)
    BM, BN = tile
    m = oracle.block_map(P, R, ps.B, ps.S, BM, BN)
    union = pairwise_union_mask(ps.B, ps.S, pl)
    for b in range(ps.B):
        np.testing.assert_array_equal(m["cls"][b], _brute_cls(union[b], ps.S, BM, BN))
        # list structure: full ascending, partial ascending, -1 fill
        for qt in range(m["nqt"]):
            nf, np_ = m["q2k_cnt"][b, qt]
            row = m["q2k_idx"][b, qt]
            assert list(row[:nf]) == sorted(k for k in range(m["nkt"]) if m["cls"][b, qt, k] == 2)
            assert list(row[nf:nf + np_]) == sorted(k for k in range(m["nkt"]) if m["cls"][b, qt, k] == 1)
            assert (row[nf + np_:] == -1).all()
    assert m["totals"].sum() == ps.B * m["nqt"] * m["nkt"]


def test_equal_length_proxy_tile_counts():
    """p1's score-size proxy at p = r = 1024: (p+2r)^2 / 2(p+r)^2 = 1.125.
    With 128-token tiles the dense packed map has 24*24 = 576 tiles and the
    two dense pairwise rows 2*16*16 = 512.  Sparse packed: the strict lower
    triangles of prompt / chosen / rejected (3*28) plus both responses
    against the prompt (2*8*8) are full, the 24 diagonal tiles are partial,
    and the upper triangle (276) plus rejected-vs-chosen (64) are skipped."""
    P, R = descriptors([(0, 0, 1024, (1024, 1024))])
    m = oracle.block_map(P, R, 1, 3072, 128, 128)
    assert m["nqt"] * m["nkt"] == 576
    Pp, Rp = descriptors([(0, 0, 1024, (1024,)), (1, 0, 1024, (1024,))])
    mp = oracle.block_map(Pp, Rp, 2, 2048, 128, 128)
    assert mp["B"] * mp["nqt"] * mp["nkt"] == 512
    assert 576 / 512 == 1.125
    assert m["totals"].tolist() == [3 * 28 + 2 * 64, 24, 276 + 64]
    assert (m["cls"][0, 16:24, 8:16] == 0).all()


def test_windows_tiny_pack_hand_values():
    P, R = descriptor_arrays(make_packset(1))
    m = oracle.block_map(P, R, 1, 144, 64, 64)
    w = m["tok_win"][0]
    assert w[10].tolist() == [0, 0, 0, 144]     # prompt token: keys [0, 10], seen by all later rows
    assert w[70].tolist() == [0, 0, 0, 96]      # chosen: one run [0, 70]; seen until chosen ends
    assert w[100].tolist() == [96, 0, 64, 144]  # rejected: prompt run + own run [96, 100]


@pytest.mark.parametrize("seed", range(20))
def test_windows_rebuild_mask(seed):
    rng = np.random.default_rng(300 + seed)
    ps = random_packset(rng, B=2, S=int(rng.integers(1, 60)), max_len=10)
    P, R = descriptor_arrays(ps)
    pk, br, _ = oracle.token_ids(P, R, ps.B, ps.S)
    S = ps.S
    for b in range(ps.B):
        mk = oracle.attention_mask(pk, br, row=b)
        w = oracle.token_windows(mk)
        i = np.arange(S)[:, None]
        j = np.arange(S)[None, :]
        from_rows = (j <= i) & ((j >= w[:, 0:1]) | ((j >= w[:, 1:2]) & (j < w[:, 2:3])))
        from_cols = (j <= i) & (i < w[None, :, 3])
        np.testing.assert_array_equal(from_rows, mk)
        np.testing.assert_array_equal(from_cols, mk)


def test_status_propagates_to_map():
    P, R = descriptors([(0, 0, 5, (6,))])
    m = oracle.block_map(P, R, 1, 10, 4, 4)
    assert m["status"].tolist() == [oracle.STATUS["bounds"], 0]
