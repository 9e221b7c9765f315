"""Aligned position ids and log-prob gather rows of a packed batch, by a
plain walk over the pack descriptors.  Test infrastructure: only the tests,
the smoke check and the benchmark's CPU baseline use it.

What the pages fix:
- "DPO Preference Packing: Dense Masks and Sparse Execution", section
  "Layout requirements": response tokens get the position ids they would
  have in their own prompt + response sequence, and the log-prob of a
  response token is read from the logits of the token before it in that
  sequence.  For a response's first token that is the last prompt token,
  not the physically preceding token (the end of the other branch).
- "Pack training sequences to reduce padding waste", sections "Decide what
  should happen at target boundaries" and "Position IDs need an explicit
  policy": no next-token target crosses the boundary between packed
  examples, and positions restart at each example.

Outputs for token s of row b (descriptor format as in oracle.segments):
    pos_ids[b, s]   prompt token j -> j; token t of a response -> prompt_len + t;
                    0 for pad.
    src_row[b, s]   index within the row of the token whose logits predict
                    token s: s - 1 inside a prompt or a response, the last
                    prompt token for a response's first token, -1 when there
                    is none (a pack's first token, a response's first token
                    after an empty prompt, pad).
    loss_mask[b, s] 1 for a response token with a predicting row (the terms
                    of that response's log-prob), else 0.
"""
from __future__ import annotations

import numpy as np

from .segments import _check


def positions(packs, resp_len, B, S):
    """(pos_ids int32 [B,S], src_row int32 [B,S], loss_mask uint8 [B,S], status).

    status = (code, pack) as in oracle.segments.token_ids; on an error the
    arrays are None (the device writes nothing then)."""
    status = _check(packs, resp_len, B, S)
    if status[0] != 0:
        return None, None, None, status
    pos = np.zeros((B, S), dtype=np.int32)
    src = np.full((B, S), -1, dtype=np.int32)
    mask = np.zeros((B, S), dtype=np.uint8)
    for row, start, plen, nresp, rfirst in np.asarray(packs, dtype=np.int64).reshape(-1, 5):
        row, start, plen = int(row), int(start), int(plen)
        for j in range(plen):  # the prompt: an ordinary sequence starting at position 0
            s = start + j
            pos[row, s] = j
            src[row, s] = s - 1 if j >= 1 else -1
        rs = start + plen
        for k in range(int(nresp)):
            r = int(resp_len[int(rfirst) + k])
            for t in range(r):  # response k continues the prompt
                s = rs + t
                pos[row, s] = plen + t
                if t >= 1:
                    src[row, s] = s - 1
                else:
                    src[row, s] = start + plen - 1 if plen >= 1 else -1
                mask[row, s] = 1 if src[row, s] >= 0 else 0
            rs += r
    return pos, src, mask, status
