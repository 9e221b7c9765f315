"""Pins of the oracle's segment ids and mask (CPU only)."""
import numpy as np
import pytest

import oracle
from oracle_pins import (closed_form_count, descriptors, pairwise_union_mask,
                         small_single_packs)
from workloads.generate import descriptor_arrays, make_packset, random_packset


def _oracle_mask(B, S, packs_list):
    P, R = descriptors(packs_list)
    pk, br, st = oracle.token_ids(P, R, B, S)
    assert tuple(st) == (0, -1)
    return oracle.attention_mask(pk, br)


def _read_grid(path):
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    return np.array([[int(x) for x in r] for r in rows], dtype=bool)


def test_p5_worked_two_example_mask(golden_dir):
    want = _read_grid(f"{golden_dir}/p5_two_examples_6x6.txt")
    assert want.sum() == 12
    # two independent 3-token examples = two prompt-only packs
    got = _oracle_mask(1, 6, [(0, 0, 3, ()), (0, 3, 3, ())])[0]
    np.testing.assert_array_equal(got, want)
    # the same two examples as zero-prompt packs with one 3-token response
    got2 = _oracle_mask(1, 6, [(0, 0, 0, (3,)), (0, 3, 0, (3,))])[0]
    np.testing.assert_array_equal(got2, want)


@pytest.mark.parametrize("pad", [0, 1, 2])
def test_exhaustive_single_packs(pad):
    n = 0
    for p, rls in small_single_packs():
        S = max(1, p + sum(rls) + pad)
        pl = [(0, 0, p, rls)]
        got = _oracle_mask(1, S, pl)
        np.testing.assert_array_equal(got, pairwise_union_mask(1, S, pl), err_msg=str((p, rls, pad)))
        assert got.sum() == closed_form_count(pl)
        n += 1
    assert n == 425


def test_exhaustive_pack_pairs_in_one_row():
    shapes = [(p, rls) for p, rls in small_single_packs() if p <= 3 and len(rls) <= 2 and max(rls, default=0) <= 2]
    cases = 0
    for (p1, r1) in shapes:
        n1 = p1 + sum(r1)
        for (p2, r2) in shapes:
            n2 = p2 + sum(r2)
            for gap in (0, 1):
                if n1 + gap + n2 > 8:
                    continue
                pl = [(0, 0, p1, r1), (0, n1 + gap, p2, r2)]
                S = max(1, n1 + gap + n2)
                got = _oracle_mask(1, S, pl)
                np.testing.assert_array_equal(got, pairwise_union_mask(1, S, pl))
                cases += 1
    assert cases > 500


@pytest.mark.parametrize("seed", range(40))
def test_random_pack_sets(seed):
    rng = np.random.default_rng(seed)
    ps = random_packset(rng, B=3, S=int(rng.integers(1, 90)), max_len=12)
    pl = [(p.row, p.start, p.prompt_len, p.resp_lens) for p in ps.packs]
    got = _oracle_mask(ps.B, ps.S, pl)
    np.testing.assert_array_equal(got, pairwise_union_mask(ps.B, ps.S, pl))
    assert got.sum() == closed_form_count(pl)


def test_negative_controls_fail():
    """A plain causal mask and a mask without pack boundaries both differ
    from the pairwise-union construction (p5 "Common packing mistakes")."""
    pl = [(0, 0, 3, (2, 2)), (0, 7, 2, (1,))]
    S = 10
    want = pairwise_union_mask(1, S, pl)
    causal = np.tril(np.ones((S, S), dtype=bool))[None]
    assert not np.array_equal(causal, want)
    P, R = descriptors(pl)
    pk, br, _ = oracle.token_ids(P, R, 1, S)
    no_boundary = oracle.attention_mask(np.where(pk >= 0, 0, -1), br)
    assert not np.array_equal(no_boundary, want)
    no_branch = oracle.attention_mask(pk, np.zeros_like(br))
    assert not np.array_equal(no_branch, want)


def test_tiny_config_counts():
    ps = make_packset(1)
    pl = [(p.row, p.start, p.prompt_len, p.resp_lens) for p in ps.packs]
    assert closed_form_count(pl) == 8904
    m = _oracle_mask(1, 144, pl)
    assert m.sum() == 8904
    # pairwise layout duplicates the prompt triangle once per extra response
    pair_count = sum(closed_form_count([(0, 0, 64, (r,))]) for r in (32, 48))
    assert pair_count == 10984 and pair_count - 8904 == 64 * 65 // 2


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [2, 3, 4, 5, "3alt"])
def test_full_config_counts_closed_form(cfg):
    ps = make_packset(cfg)
    P, R = descriptor_arrays(ps)
    pk, br, st = oracle.token_ids(P, R, ps.B, ps.S)
    assert tuple(st) == (0, -1)
    pl = [(p.row, p.start, p.prompt_len, p.resp_lens) for p in ps.packs]
    n = sum(oracle.allowed_count(oracle.attention_mask(pk, br, row=b)) for b in range(ps.B))
    assert n == closed_form_count(pl)


def test_status_codes():
    S = oracle.STATUS
    B, L = 2, 10
    ok = [(0, 0, 2, (1, 1)), (1, 0, 3, ())]
    P, R = descriptors(ok)
    assert tuple(oracle.token_ids(P, R, B, L)[2]) == (0, -1)
    cases = {
        "row": [(0, 0, 2, ()), (2, 0, 1, ())],
        "negative": [(0, 0, -1, ())],
        "bounds": [(0, 0, 5, (6,))],
        "order": [(0, 4, 2, ()), (0, 5, 1, ())],
    }
    for name, pl in cases.items():
        P, R = descriptors(pl)
        code, bad = oracle.token_ids(P, R, B, L)[2]
        assert code == S[name], name
        assert bad == len(pl) - 1
    P, R = descriptors([(0, 0, 2, (1,))])
    P[0, 4] = 5  # resp_first out of range
    assert oracle.token_ids(P, R, B, L)[2] == (S["resp_range"], 0)
    P, R = descriptors([(0, 0, 2, (1,))])
    R[0] = -3
    assert oracle.token_ids(P, R, B, L)[2] == (S["negative"], 0)
    # descending rows are an order error
    P, R = descriptors([(1, 0, 1, ()), (0, 0, 1, ())])
    assert oracle.token_ids(P, R, B, L)[2] == (S["order"], 1)
