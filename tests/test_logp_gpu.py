"""GPU packed token log-probs vs the oracle (fp64).

Tolerance: each lane folds about V/256 logits into an fp32 online
log-sum-exp, so the relative error of the sum is at most ~(V/256) * 2^-24
(3.6e-5 at V = 151936), i.e. an absolute error of that size on the log;
TOK_ABS = 1e-4 covers it with margin.  A response sum of n terms then errs
by at most n * TOK_ABS."""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_path import api, build_map, say
from oracle_pins import descriptors
from workloads.generate import Pack, PackSet, descriptor_arrays, make_packset, random_packset

pytestmark = pytest.mark.gpu

TOK_ABS = 1e-4


def _inputs(ps, V, seed, sigma=3.0):
    g = torch.Generator().manual_seed(seed)
    logits = (torch.randn((ps.B, ps.S, V), generator=g, dtype=torch.float32) * sigma).to(torch.bfloat16)
    tokens = torch.randint(0, V, (ps.B, ps.S), generator=g, dtype=torch.int32)
    return logits, tokens


def _run(ps, logits, tokens, tile=(64, 64)):
    A = api()
    P, R = descriptor_arrays(ps)
    pd, rd = A.descriptors_to_device(P, R)
    m = A.pack_block_map(pd, rd, ps.B, ps.S, *tile)
    pos, src, mask = A.pack_positions(m)
    tok, resp = A.packed_token_logp(m, src, mask, logits.cuda().contiguous(), tokens.cuda(), pd, rd)
    torch.cuda.synchronize()
    return P, R, tok.cpu().double().numpy(), resp.cpu().double().numpy()


def _check(ps, logits, tokens, P, R, tok, resp):
    _, src, mask, _ = oracle.positions(P, R, ps.B, ps.S)
    lf = logits.float()
    want = oracle.token_logp(lambda b, r: lf[b, r].numpy(), tokens.numpy(), src, mask)
    err = float(np.abs(tok - want).max()) if tok.size else 0.0
    assert err <= TOK_ABS, err
    rw = oracle.response_logp(P, R, want)
    lens = np.asarray(R, dtype=np.float64)
    assert (np.abs(resp - rw) <= TOK_ABS * np.maximum(lens, 1)).all()
    return err


@pytest.mark.parametrize("seed", range(6))
def test_random_ragged_small_vocab(seed):
    rng = np.random.default_rng(3000 + seed)
    ps = random_packset(rng, B=int(rng.integers(1, 3)), S=int(rng.integers(8, 300)), max_packs_per_row=4,
                        max_resp=4, max_len=int(rng.integers(2, 60)))
    V = [8, 104, 1024, 4096, 2048, 512][seed]
    logits, tokens = _inputs(ps, V, seed)
    say("logp random", seed, ps.B, ps.S, V, len(ps.packs))
    P, R, tok, resp = _run(ps, logits, tokens)
    e = _check(ps, logits, tokens, P, R, tok, resp)
    say("  max abs err", e)


def test_tiny_config_marker_logits():
    """Every response token scores the marker of its own pairwise predecessor's row."""
    ps = make_packset(1)
    V = 104
    logits = torch.zeros((1, ps.S, V))
    for r in range(ps.S):
        logits[0, r, (3 * r + 1) % V] = 8.0
    P, R = descriptor_arrays(ps)
    _, src, mask, _ = oracle.positions(P, R, ps.B, ps.S)
    tokens = torch.zeros((1, ps.S), dtype=torch.int32)
    tokens[0] = torch.from_numpy(((3 * np.maximum(src[0], 0) + 1) % V).astype(np.int32))
    P, R, tok, resp = _run(ps, logits.to(torch.bfloat16), tokens)
    hit = 8.0 - math.log(math.exp(8.0) + V - 1)
    assert np.abs(tok[0][mask[0] == 1] - hit).max() <= TOK_ABS
    assert (tok[0][mask[0] == 0] == 0).all()
    assert np.abs(resp - np.array([32 * hit, 48 * hit])).max() <= 32 * TOK_ABS


def test_full_vocab_sampled():
    """The Qwen3-8B-shaped packs with a 151936-token vocabulary (4.4 GB of
    logits); the oracle checks sampled tokens and every response sum's
    sampled terms."""
    ps = make_packset(2)
    V = 151936
    g = torch.Generator(device="cuda").manual_seed(11)
    logits = (torch.randn((ps.B, ps.S, V), generator=g, device="cuda", dtype=torch.float32) * 2.5).to(torch.bfloat16)
    tokens = torch.randint(0, V, (ps.B, ps.S), generator=g, device="cuda", dtype=torch.int32)
    A = api()
    P, R = descriptor_arrays(ps)
    pd, rd = A.descriptors_to_device(P, R)
    m = A.pack_block_map(pd, rd, ps.B, ps.S, 32, 64)
    pos, src, mask = A.pack_positions(m)
    tok, resp = A.packed_token_logp(m, src, mask, logits, tokens, pd, rd)
    torch.cuda.synchronize()
    say("logp full vocab", ps.B, ps.S, V)
    _, osrc, omask, _ = oracle.positions(P, R, ps.B, ps.S)
    rng = np.random.default_rng(5)
    cand = np.argwhere(omask == 1)
    pick = cand[rng.choice(len(cand), size=48, replace=False)]
    where = np.zeros_like(omask, dtype=bool)
    where[pick[:, 0], pick[:, 1]] = True
    rows = {}
    def row(b, r):
        if (b, r) not in rows:
            rows[(b, r)] = logits[b, r].float().cpu().numpy()
        return rows[(b, r)]
    want = oracle.token_logp(row, tokens.cpu().numpy(), osrc, omask, where=where)
    got = tok.cpu().double().numpy()
    err = float(np.abs(got[where] - want[where]).max())
    say("  sampled max abs err", err)
    assert err <= TOK_ABS
    # each response sum equals the sum of its GPU token terms in fp64 (and is finite)
    tk = tok.cpu().double().numpy()
    rs = oracle.response_logp(P, R, tk)
    assert np.isfinite(resp.cpu().numpy()).all()
    assert (np.abs(resp.cpu().double().numpy() - rs) <= 1e-5 * np.abs(rs) + 1e-3).all()
    del logits


def test_leading_masked_logits():
    """Rows whose leading logits are -inf (masked vocabulary entries): every
    lane's first chunks see nothing but -inf, which must not turn the running
    log-sum-exp into NaN.  The first 4096 of V = 8192 logits of every row
    are -inf; tokens in the masked part get -inf, the others the oracle's
    value."""
    ps = make_packset(1)
    V = 8192
    logits, tokens = _inputs(ps, V, 4)
    logits[:, :, :4096] = float("-inf")
    tokens[0, ::2] = 0  # masked token id
    P, R = descriptor_arrays(ps)
    A = api()
    pd, rd = A.descriptors_to_device(P, R)
    m = A.pack_block_map(pd, rd, ps.B, ps.S, 64, 64)
    pos, src, mask = A.pack_positions(m)
    tok, _ = A.packed_token_logp(m, src, mask, logits.cuda().contiguous(), tokens.cuda(), pd, rd)
    torch.cuda.synchronize()
    got = tok.cpu().double().numpy()
    _, osrc, omask, _ = oracle.positions(P, R, ps.B, ps.S)
    lf = logits.float()
    want = oracle.token_logp(lambda b, r: lf[b, r].numpy(), tokens.numpy(), osrc, omask)
    say("logp leading -inf logits", int(np.isnan(got).sum()))
    assert not np.isnan(got).any()
    inf = np.isneginf(want)
    assert inf.any() and (~inf & (omask == 1)).any()
    assert np.array_equal(np.isneginf(got), inf)
    assert float(np.abs(got[~inf] - want[~inf]).max()) <= TOK_ABS


def test_bad_token_and_invalid_map():
    A = api()
    ps = make_packset(1)
    V = 64
    logits, tokens = _inputs(ps, V, 1)
    tokens[0, 70] = V + 5  # a response token: its log-prob becomes NaN
    P, R, tok, resp = _run(ps, logits, tokens)
    assert math.isnan(tok[0, 70]) and not np.isnan(tok[0, 69])
    P2, R2 = descriptors([(0, 0, 4, (3,)), (0, 2, 1, ())])
    pd, rd = A.descriptors_to_device(P2, R2)
    bad = A.pack_block_map(pd, rd, 1, 16, 64, 64)
    src = torch.zeros((1, 16), dtype=torch.int32, device="cuda")
    mask = torch.ones((1, 16), dtype=torch.uint8, device="cuda")
    out = torch.full((1, 16), 7.0, device="cuda")
    lg = torch.zeros((1, 16, 8), dtype=torch.bfloat16, device="cuda")
    A.packed_token_logp(bad, src, mask, lg, torch.zeros((1, 16), dtype=torch.int32, device="cuda"),
                        out=(out, None))
    torch.cuda.synchronize()
    assert (out == 7.0).all()
