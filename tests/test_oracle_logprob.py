"""Pins of the oracle's packed token log-probs (CPU only)."""
import math

import numpy as np
import pytest

import oracle
from oracle_pins import descriptors
from workloads.generate import descriptor_arrays, make_packset, random_packset


@pytest.mark.parametrize("V", [1, 7, 1024])
def test_uniform_logits_give_minus_log_V(V):
    x = np.full(V, 3.25)
    assert abs(oracle.row_logsumexp(x) - (3.25 + math.log(V))) < 1e-12
    tok = np.zeros((1, 1), dtype=np.int32)
    got = oracle.token_logp(lambda b, r: x, tok, np.zeros((1, 1), np.int32), np.ones((1, 1), np.uint8))
    assert abs(got[0, 0] + math.log(V)) < 1e-12


@pytest.mark.parametrize("a,b,V", [(5.0, -1.0, 10), (-2.0, 0.5, 3), (30.0, 0.0, 151936)])
def test_two_level_closed_form(a, b, V):
    """One logit a, the other V-1 equal to b: p(a) = e^a / (e^a + (V-1) e^b)."""
    x = np.full(V, b)
    x[V // 2] = a
    norm = math.log(math.exp(a) + (V - 1) * math.exp(b))
    lse = oracle.row_logsumexp(x)
    assert abs(lse - norm) < 1e-10 * max(1.0, abs(norm))
    assert abs((x[V // 2] - lse) - (a - norm)) < 1e-10
    assert abs((x[0] - lse) - (b - norm)) < 1e-10


@pytest.mark.parametrize("k,V", [(8, 16), (4096, 8192), (1, 2)])
def test_masked_logits_closed_form(k, V):
    """Logits masked to -inf drop out of the normaliser: with k of them and
    V - k equal finite logits c, a finite token has log-prob -ln(V - k) and
    a masked token -inf."""
    x = np.full(V, 1.5)
    x[:k] = -np.inf
    assert abs(oracle.row_logsumexp(x) - (1.5 + math.log(V - k))) < 1e-12
    tok = np.array([[V - 1, 0]], dtype=np.int32)
    got = oracle.token_logp(lambda b, r: x, tok, np.zeros((1, 2), np.int32), np.ones((1, 2), np.uint8))
    assert abs(got[0, 0] + math.log(V - k)) < 1e-12
    assert got[0, 1] == -np.inf


def test_shift_invariance_and_normalisation():
    rng = np.random.default_rng(3)
    x = rng.normal(0, 3, size=5000)
    lse = oracle.row_logsumexp(x)
    assert abs(np.exp(x - lse).sum() - 1.0) < 1e-12
    for c in (-1e4, 7.5, 1e4):  # large offsets stay finite (max subtracted first)
        assert abs(oracle.row_logsumexp(x + c) - (lse + c)) < 1e-9 * max(1.0, abs(c))


def _pairwise_predecessor(ps):
    """Independent: predecessor of each response token in its own
    [prompt | response k] sequence (None for a sequence's first token)."""
    pred = {}
    for p in ps.packs:
        prompt = list(range(p.start, p.start + p.prompt_len))
        rs = p.start + p.prompt_len
        for r in p.resp_lens:
            seq = prompt + list(range(rs, rs + r))
            for i in range(p.prompt_len, len(seq)):
                pred[(p.row, seq[i])] = seq[i - 1] if i >= 1 else None
            rs += r
    return pred


@pytest.mark.parametrize("cfg", [1, "rand0", "rand1"])
def test_gather_reads_the_predicting_row(cfg):
    """Marker logits: row r puts 8 on token (3r + 1) mod V, 0 elsewhere.  Each
    response token's id is set to its own pairwise predecessor's marker, so a
    token scores the high value exactly when the gather row is that
    predecessor ("DPO Preference Packing: Dense Masks and Sparse Execution",
    section "Layout requirements": a response's first token is predicted
    from the final prompt row)."""
    ps = make_packset(1) if cfg == 1 else random_packset(np.random.default_rng(int(cfg[-1])), 2, 120, max_len=20)
    V = 97
    P, R = descriptor_arrays(ps)
    pos, src, mask, st = oracle.positions(P, R, ps.B, ps.S)
    pred = _pairwise_predecessor(ps)
    tokens = np.zeros((ps.B, ps.S), dtype=np.int32)
    for (b, s), r in pred.items():
        if r is not None:
            tokens[b, s] = (3 * r + 1) % V

    def row(b, r):
        x = np.zeros(V)
        x[(3 * r + 1) % V] = 8.0
        return x

    got = oracle.token_logp(row, tokens, src, mask)
    hit = 8.0 - math.log(math.exp(8.0) + V - 1)
    n_terms = sum(1 for r in pred.values() if r is not None)
    assert int(mask.sum()) == n_terms
    assert np.allclose(got[mask == 1], hit, atol=1e-12)
    assert (got[mask == 0] == 0).all()
    resp = oracle.response_logp(P, R, got)
    i = 0
    for p in ps.packs:
        for r in p.resp_lens:
            want = hit * (r if p.prompt_len >= 1 else max(r - 1, 0))
            assert abs(resp[i] - want) < 1e-9, (p, r)
            i += 1
    if cfg == 1:  # a one-position shift reads the rejected start from row 95: a miss
        naive = (3 * 95 + 1) % V
        assert naive != tokens[0, 96] and src[0, 96] == 63
