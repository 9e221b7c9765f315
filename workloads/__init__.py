"""Seeded synthetic workloads for packed branch-aware attention.

This module only draws numbers and lays tokens out; it holds none of the
attention or masking arithmetic.  Both the fp64 oracle tests and the HIP path
(tests and bench) take their inputs from here, so the two sides see the very
same descriptors and bf16 tensors.

Layout of one pack (p1 "Layout requirements": prompt + chosen + rejected,
generalised to K responses in p2 section 3.1): the prompt tokens, then each
response's tokens, contiguous inside one row.  Several packs may share a row,
separated as by cumulative sequence lengths (p3 "The correct implementation").
"""
from .generate import (  # noqa: F401
    Pack, PackSet, Workload, CONFIG_NAMES,
    lognormal_length, make_packset, make_workload, pairwise_packset,
    pairwise_tensors, descriptor_arrays, pad_to_len,
)
