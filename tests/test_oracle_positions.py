"""Pins of the oracle's aligned positions and log-prob gather rows (CPU only)."""
import numpy as np
import pytest

import oracle
from oracle_pins import descriptors, small_single_packs
from workloads.generate import descriptor_arrays, make_packset, random_packset


def _positions(B, S, packs_list):
    P, R = descriptors(packs_list)
    pos, src, mask, st = oracle.positions(P, R, B, S)
    assert tuple(st) == (0, -1)
    return pos, src, mask


def _golden_cases(path):
    cases, cur = [], None
    for line in open(path):
        if not line.strip() or line.startswith("#"):
            continue
        f = line.split()
        if f[0] == "case":
            cur = {"prompts": [int(x) for x in f[1:]]}
            cases.append(cur)
        else:
            cur[f[0]] = [int(x) for x in f[1:]]
    return cases


def test_p5_positions_and_target_boundaries(golden_dir):
    """Positions restart per example and no target crosses the boundary
    ("Pack training sequences to reduce padding waste", sections on position
    IDs and on target boundaries): the pages' own worked tables."""
    cases = _golden_cases(f"{golden_dir}/p5_positions_targets.txt")
    assert len(cases) == 2
    for c in cases:
        packs, start = [], 0
        for n in c["prompts"]:
            packs.append((0, start, n, ()))
            start += n
        pos, src, _ = _positions(1, start, packs)
        if "positions" in c:
            assert pos[0].tolist() == c["positions"]
        if "valid" in c:
            # a row is a valid input when its logits predict a token of the same example
            valid = [int((src[0] == i).any()) for i in range(start)]
            assert valid == c["valid"]


def test_p1_branch_start_reads_the_last_prompt_row():
    """Tiny pack (prompt 64, chosen 32, rejected 48), rows 0-143: the
    responses begin at rows 64 and 96, both at position id 64, and the
    source row of each of those two tokens is 63.  Asserted against the
    plain shift src = s - 1, which gives 95 for row 96 ("DPO Preference
    Packing: Dense Masks and Sparse Execution", section "Layout
    requirements")."""
    ps = make_packset(1, 0)
    P, R = descriptor_arrays(ps)
    pos, src, mask, st = oracle.positions(P, R, ps.B, ps.S)
    assert tuple(st) == (0, -1)
    assert pos[0, 64] == 64 and pos[0, 96] == 64 and pos[0, 143] == 64 + 47
    assert src[0, 64] == 63 and src[0, 96] == 63
    assert src[0, 97] == 96 and src[0, 65] == 64 and src[0, 1] == 0 and src[0, 0] == -1
    naive_shift = np.arange(ps.S) - 1
    assert naive_shift[96] == 95 != src[0, 96]
    assert mask[0].sum() == 32 + 48 and mask[0, :64].sum() == 0


def _pairwise_pins(B, S, packs_list):
    """Independent construction: each response k of a pack as its own
    sequence [prompt | response k] (the pairwise layout), whose positions
    are 0.. and whose next-token predecessor is simply the previous element.
    Returns per-token expected (pos, src, mask) for tokens of the packs."""
    pos = np.zeros((B, S), dtype=np.int64)
    src = np.full((B, S), -1, dtype=np.int64)
    mask = np.zeros((B, S), dtype=np.int64)
    for row, start, p, rls in packs_list:
        prompt = list(range(start, start + p))
        seqs = []
        rs = start + p
        for r in rls:
            seqs.append((prompt, list(range(rs, rs + r))))
            rs += r
        if not rls:
            seqs.append((prompt, []))
        for pr, resp in seqs:
            seq = pr + resp
            for idx, s in enumerate(seq):
                pos[row, s] = idx
                src[row, s] = seq[idx - 1] if idx >= 1 else -1
                mask[row, s] = 1 if (s in resp and idx >= 1) else 0
    return pos, src, mask


def test_exhaustive_single_packs_match_pairwise():
    n = 0
    for p, rls in small_single_packs():
        for pad in (0, 2):
            S = max(1, p + sum(rls) + pad)
            pl = [(0, 0, p, rls)]
            got = _positions(1, S, pl)
            want = _pairwise_pins(1, S, pl)
            for g, w_, name in zip(got, want, ("pos", "src", "mask")):
                np.testing.assert_array_equal(g.astype(np.int64), w_, err_msg=f"{name} {(p, rls, pad)}")
            n += 1
    assert n == 850


@pytest.mark.parametrize("seed", range(6))
def test_random_pack_sets_match_pairwise_and_closed_form(seed):
    rng = np.random.default_rng(100 + seed)
    ps = random_packset(rng, 3, 160)
    pl = [(p.row, p.start, p.prompt_len, p.resp_lens) for p in ps.packs]
    got = _positions(ps.B, ps.S, pl)
    want = _pairwise_pins(ps.B, ps.S, pl)
    for g, w_ in zip(got, want):
        np.testing.assert_array_equal(g.astype(np.int64), w_)
    # closed form: every response token has a predictor except the first one after an empty prompt
    count = sum(sum(r if p.prompt_len >= 1 else max(r - 1, 0) for r in p.resp_lens) for p in ps.packs)
    assert int(got[2].sum()) == count
    # pad: position 0, no predictor, not in the loss
    covered = np.zeros((ps.B, ps.S), dtype=bool)
    for p in ps.packs:
        covered[p.row, p.start:p.start + p.length] = True
    assert (got[0][~covered] == 0).all() and (got[1][~covered] == -1).all() and (got[2][~covered] == 0).all()


def test_invalid_descriptors_give_no_output():
    P, R = descriptors([(0, 0, 4, (3,)), (0, 2, 1, ())])  # overlapping packs
    pos, src, mask, st = oracle.positions(P, R, 1, 16)
    assert st[0] != 0 and pos is None and src is None and mask is None
