"""fp64 CPU oracle for packed branch-aware causal attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The library and its
Python binding never do, and this package imports nothing from them: the two
share no code, headers, tables or helpers.  Inputs come from the seeded
generators in `workloads`, which hold no attention arithmetic.

What it computes is the plain definition (p1 "Dense and sparse execution":
block skipping only drops work whose contribution is exactly zero, so the
method equals ordinary masked softmax attention):

  segments.token_ids     per-token pack index and branch id from descriptors
  segments.attention_mask the branch-aware, pack-bounded causal mask
  segments.token_windows per-token runs of the mask (query and key views)
  segments.block_map     brute-force tile classification and visit lists
  attention.attn_fwd / attn_bwd   dense fp64 masked attention and its naive
                         backward (softmax Jacobian), per row and q-head
  positions.positions    aligned position ids, log-prob gather rows and the
                         response loss mask from descriptors
  logprob.token_logp / response_logp   log-softmax at the gather rows and
                         per-response sums
  groupdpo               group preference objectives over packs of K
                         responses and their surrogate coefficients
  rope                   rotary embedding at the packed (branch-aligned)
                         position ids, and its inverse for gradients

Every function is pinned in tests/ against facts the pages or mathematics
fix (worked masks, closed-form counts, brute force, finite differences,
packed-vs-pairwise equivalence, library special cases).
"""
from .segments import (  # noqa: F401
    STATUS, token_ids, attention_mask, attention_mask_rows, token_windows, block_map, allowed_count,
)
from .attention import (  # noqa: F401
    attn_fwd, attn_bwd, attn_fwd_rows, attn_dq_rows, attn_dkdv_rows, attn_bwd_sampled, useful_flops,
)
from .positions import positions  # noqa: F401
from .logprob import row_logsumexp, token_logp, response_logp  # noqa: F401
from . import groupdpo  # noqa: F401
from . import rope  # noqa: F401
