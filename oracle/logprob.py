"""Packed token log-probs and per-response sums, in fp64.  Test
infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use it.

"DPO Preference Packing: Dense Masks and Sparse Execution", section "Layout
requirements": a response's log-prob is gathered from the logits that
predict each of its tokens, the first one from the final prompt row.  With
the gather rows of oracle.positions (src_row) and the response loss mask,
the log-prob of token s is the log-softmax of its predicting row's logits
at its token id:

    tok_logp[b, s] = logits[b, r, y] - log sum_v exp(logits[b, r, v]),
                     r = src_row[b, s], y = tokens[b, s]      (loss_mask = 1)
    tok_logp[b, s] = 0                                        (loss_mask = 0)

and the log-prob of response k of a pack is the sum of tok_logp over that
response's tokens (the per-sequence quantity DPO compares between the
chosen and the rejected response).  The log-sum-exp is taken with the row
max subtracted first (exact in fp64 for bf16 logits).
"""
from __future__ import annotations

import numpy as np


def row_logsumexp(x):
    """log sum_v exp(x_v) of a 1-D array, in fp64 (max subtracted first)."""
    x = np.asarray(x, dtype=np.float64)
    m = x.max()
    return m + np.log(np.exp(x - m).sum())


def token_logp(logits_row_fn, tokens, src_row, loss_mask, where=None):
    """tok_logp [B, S] fp64.  `logits_row_fn(b, r)` returns row r of batch
    row b's logits as a 1-D array (so that huge vocabularies need not be
    materialised on the host); `where` optionally restricts the computation
    to a boolean [B, S] subset (other entries are NaN)."""
    tokens = np.asarray(tokens)
    src_row = np.asarray(src_row)
    loss_mask = np.asarray(loss_mask)
    B, S = tokens.shape
    out = np.zeros((B, S), dtype=np.float64)
    if where is not None:
        out[~where] = np.nan
    for b in range(B):
        for s in range(S):
            if where is not None and not where[b, s]:
                continue
            if not loss_mask[b, s]:
                continue
            x = np.asarray(logits_row_fn(b, int(src_row[b, s])), dtype=np.float64)
            out[b, s] = x[int(tokens[b, s])] - row_logsumexp(x)
    return out


def response_logp(packs, resp_len, tok_logp):
    """Sum of tok_logp over each response's tokens, indexed like resp_len."""
    R = len(resp_len)
    out = np.zeros(R, dtype=np.float64)
    for row, start, plen, nresp, rfirst in np.asarray(packs, dtype=np.int64).reshape(-1, 5):
        rs = int(start) + int(plen)
        for k in range(int(nresp)):
            r = int(resp_len[int(rfirst) + k])
            out[int(rfirst) + k] = float(np.sum(tok_logp[int(row), rs:rs + r]))
            rs += r
    return out
