"""Segment ids, the mask, per-token windows and the block map, by brute force.

Descriptor format (one int32 row per pack, sorted by (row, start)):
    (row, start, prompt_len, n_resp, resp_first)
plus the concatenated response lengths `resp_len`.  Pack p covers tokens
[start, start + prompt_len + sum(resp_len[resp_first : resp_first + n_resp]))
of row `row`: its prompt first, then each response (p1 "Layout
requirements"; K responses after one prompt as in p2 section 3.1; several
packs per row as in p3 "The correct implementation").
"""
from __future__ import annotations

import numpy as np

# Device status codes of the descriptor checks (the same numbers the C ABI
# documents for the map's status word).  status = (code, first bad pack).
STATUS = {
    "ok": 0,
    "row": 1,        # row outside [0, B)
    "negative": 2,   # negative start, prompt_len, n_resp or a response length
    "resp_range": 3, # resp_first / n_resp outside resp_len[]
    "bounds": 4,     # pack runs past the end of its row (start + len > S)
    "order": 5,      # not sorted by (row, start) or overlaps the previous pack
}


def _check(packs, resp_len, B, S):
    """First offending pack and its code, checks in the order listed above."""
    prev_row, prev_end = -1, 0
    R = len(resp_len)
    for p, (row, start, plen, nresp, rfirst) in enumerate(np.asarray(packs, dtype=np.int64).reshape(-1, 5)):
        if row < 0 or row >= B:
            return STATUS["row"], p
        if start < 0 or plen < 0 or nresp < 0:
            return STATUS["negative"], p
        if rfirst < 0 or rfirst + nresp > R:
            return STATUS["resp_range"], p
        rl = np.asarray(resp_len[rfirst:rfirst + nresp], dtype=np.int64)
        if (rl < 0).any():
            return STATUS["negative"], p
        end = start + plen + int(rl.sum())
        if end > S:
            return STATUS["bounds"], p
        if row < prev_row or (row == prev_row and start < prev_end):
            return STATUS["order"], p
        prev_row, prev_end = row, end
    return STATUS["ok"], -1


def token_ids(packs, resp_len, B, S):
    """Per-token pack index and branch id.

    tok_pack[b, s]   = index of the pack covering token s of row b, else -1 (pad)
    tok_branch[b, s] = 0 in the prompt, k + 1 in response k, 0 for pad
    Returns (tok_pack, tok_branch, status) with status = (code, pack) and
    (0, -1) when the descriptors are valid; on an error the id arrays are
    all pad.
    """
    tok_pack = np.full((B, S), -1, dtype=np.int32)
    tok_branch = np.zeros((B, S), dtype=np.int32)
    code, bad = _check(packs, resp_len, B, S)
    if code != 0:
        return tok_pack, tok_branch, (code, bad)
    for p, (row, start, plen, nresp, rfirst) in enumerate(np.asarray(packs, dtype=np.int64).reshape(-1, 5)):
        tok_pack[row, start:start + plen] = p
        pos = start + plen
        for k in range(nresp):
            r = int(resp_len[rfirst + k])
            tok_pack[row, pos:pos + r] = p
            tok_branch[row, pos:pos + r] = k + 1
            pos += r
    return tok_pack, tok_branch, (0, -1)


def attention_mask(tok_pack, tok_branch, row=None):
    """allowed[b, i, j]: query i may attend key j.

    Same pack (pack boundaries act like cumulative sequence lengths, p3 and
    p5 "allow = same example AND key position <= query position"), causal
    in physical order, and a key inside a response is visible only to
    queries of that same response (p1 "Layout requirements": each response
    sees the shared prompt and its own earlier tokens, never a sibling).
    Pad queries see nothing.
    """
    pk = tok_pack if row is None else tok_pack[row:row + 1]
    br = tok_branch if row is None else tok_branch[row:row + 1]
    S = pk.shape[1]
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    same_pack = (pk[:, :, None] == pk[:, None, :]) & (pk[:, :, None] >= 0)
    causal = (j <= i)[None]
    branch_ok = (br[:, None, :] == 0) | (br[:, None, :] == br[:, :, None])
    m = same_pack & causal & branch_ok
    return m if row is None else m[0]


def attention_mask_rows(tok_pack, tok_branch, row, queries):
    """allowed[i, j] of batch row `row` for the listed query positions only
    (the same rule as attention_mask, without forming the S x S matrix)."""
    pk, br = tok_pack[row], tok_branch[row]
    q = np.asarray(queries)
    S = pk.shape[0]
    j = np.arange(S)[None, :]
    same_pack = (pk[None, :] == pk[q][:, None]) & (pk[q][:, None] >= 0)
    causal = j <= q[:, None]
    branch_ok = (br[None, :] == 0) | (br[None, :] == br[q][:, None])
    return same_pack & causal & branch_ok


def allowed_count(mask) -> int:
    return int(np.count_nonzero(mask))


def _runs(v):
    """[start, end) of each run of True in a 1-D bool array."""
    d = np.diff(np.concatenate(([0], v.astype(np.int8), [0])))
    return list(zip(np.flatnonzero(d == 1), np.flatnonzero(d == -1)))


def token_windows(mask_b):
    """Per-token windows of one row's mask, read off the mask itself.

    Query view of token i: its allowed keys are [pre_lo, pre_hi) U [kv_lo, i].
    The last run of allowed keys ends at i and starts at kv_lo; when there is
    an earlier, separate run (the prompt seen from a later response) it is
    [pre_lo, pre_hi), otherwise (0, 0).  A pad query has kv_lo = i + 1.
    Key view of token j: the queries that see it are [j, q_end); q_end = j for
    a pad key.  Returns int32 [S, 4] = (kv_lo, pre_lo, pre_hi, q_end) and
    raises if the mask does not have this shape.
    """
    S = mask_b.shape[0]
    win = np.zeros((S, 4), dtype=np.int32)
    for i in range(S):
        runs = _runs(mask_b[i])
        if not runs:
            win[i, 0] = i + 1
        else:
            if len(runs) > 2 or runs[-1][1] != i + 1:
                raise AssertionError(f"row {i}: runs {runs}")
            win[i, 0] = runs[-1][0]
            if len(runs) == 2:
                win[i, 1], win[i, 2] = runs[0]
        cruns = _runs(mask_b[:, i])
        if not cruns:
            win[i, 3] = i
        else:
            if len(cruns) != 1 or cruns[0][0] != i:
                raise AssertionError(f"col {i}: runs {cruns}")
            win[i, 3] = cruns[0][1]
    return win


def block_map(packs, resp_len, B, S, BM, BN):
    """Tile classification and visit lists by counting mask ones per tile.

    The token axis is extended to nqt*BM (queries) and nkt*BN (keys) with pad
    tokens.  For tile (qt, kt) with c allowed pairs: cls = 2 (full) if
    c = BM*BN, 0 (skip) if c = 0, else 1 (partial).  Fully masked tiles are
    the ones a block mask skips (p1 "Dense and sparse execution").
    q2k lists, per (b, qt): the full kt ascending, then the partial kt
    ascending, then -1; counts (n_full, n_partial).  k2q is the same per
    (b, kt) over qt.  totals = (n_full, n_partial, n_skip).
    q_order: the flat query-tile indices b*nqt + qt sorted by visit count
    (n_full + n_partial) descending, ties by index ascending; k_order the
    same over b*nkt + kt.  (A work order, longest lists first; it does not
    change what is computed.)
    """
    nqt = -(-S // BM)
    nkt = -(-S // BN)
    tok_pack, tok_branch, status = token_ids(packs, resp_len, B, S)
    out = {
        "B": B, "S": S, "block_m": BM, "block_n": BN, "nqt": nqt, "nkt": nkt,
        "tok_pack": tok_pack, "tok_branch": tok_branch, "status": np.asarray(status, dtype=np.int32),
    }
    if status[0] != 0:
        return out
    cls = np.zeros((B, nqt, nkt), dtype=np.uint8)
    win = np.zeros((B, S, 4), dtype=np.int32)
    for b in range(B):
        m = attention_mask(tok_pack, tok_branch, row=b)
        win[b] = token_windows(m)
        big = np.zeros((nqt * BM, nkt * BN), dtype=bool)
        big[:S, :S] = m
        cnt = big.reshape(nqt, BM, nkt, BN).sum(axis=(1, 3))
        cls[b] = np.where(cnt == BM * BN, 2, np.where(cnt == 0, 0, 1))
    q2k_cnt = np.zeros((B, nqt, 2), dtype=np.int32)
    q2k_idx = np.full((B, nqt, nkt), -1, dtype=np.int32)
    k2q_cnt = np.zeros((B, nkt, 2), dtype=np.int32)
    k2q_idx = np.full((B, nkt, nqt), -1, dtype=np.int32)
    for b in range(B):
        for qt in range(nqt):
            full = [kt for kt in range(nkt) if cls[b, qt, kt] == 2]
            part = [kt for kt in range(nkt) if cls[b, qt, kt] == 1]
            q2k_cnt[b, qt] = (len(full), len(part))
            q2k_idx[b, qt, :len(full) + len(part)] = full + part
        for kt in range(nkt):
            full = [qt for qt in range(nqt) if cls[b, qt, kt] == 2]
            part = [qt for qt in range(nqt) if cls[b, qt, kt] == 1]
            k2q_cnt[b, kt] = (len(full), len(part))
            k2q_idx[b, kt, :len(full) + len(part)] = full + part
    def longest_first(cnt):
        visits = cnt.reshape(-1, 2).sum(axis=1)
        keyed = sorted(range(len(visits)), key=lambda i: (-int(visits[i]), i))
        return np.asarray(keyed, dtype=np.int32)

    out.update(
        q_order=longest_first(q2k_cnt), k_order=longest_first(k2q_cnt),
        tok_win=win, cls=cls, q2k_cnt=q2k_cnt, q2k_idx=q2k_idx, k2q_cnt=k2q_cnt, k2q_idx=k2q_idx,
        totals=np.array([(cls == 2).sum(), (cls == 1).sum(), (cls == 0).sum()], dtype=np.int64),
    )
    return out
