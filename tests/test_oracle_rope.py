"""Pins of the oracle's rotary embedding (CPU only).

What fixes it: position 0 is the identity; for D = 2 it is the plane
rotation by pos (closed form); rotations preserve norms; R(a) R(b) = R(a+b)
and the inverse undoes the forward; rotated query-key dot products depend
only on the position difference (the property the packed layout needs:
a response at aligned positions scores like its own sequence); the
interleaved pairing is the rotate-half one with the head dims permuted; the
frequencies are base^(-2i/D)."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import rope as R
from oracle_pins import descriptors, rope as interleaved_helper


def _x(T=5, H=3, D=8, seed=0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((T, H, D), generator=g, dtype=torch.float64)


def test_position_zero_is_identity():
    x = _x()
    assert torch.equal(R.rope(x, [0] * 5), x)


@pytest.mark.parametrize("pos", [0, 1, 3, 17, 1000])
def test_two_dims_is_the_plane_rotation(pos):
    x = torch.tensor([[[0.6, -1.3]]], dtype=torch.float64)
    y = R.rope(x, [pos], base=10000.0)
    c, s = math.cos(pos), math.sin(pos)  # f_0 = 1
    assert abs(float(y[0, 0, 0]) - (0.6 * c + 1.3 * s)) < 1e-12
    assert abs(float(y[0, 0, 1]) - (0.6 * s - 1.3 * c)) < 1e-12


def test_frequencies():
    f = R.rope_freqs(128, 1e6)
    assert float(f[0]) == 1.0
    assert abs(float(f[32]) - 1e6 ** -0.5) < 1e-15
    assert abs(float(f[63]) - 1e6 ** (-126 / 128)) < 1e-18


def test_norm_composition_and_inverse():
    x = _x(T=6, H=2, D=16)
    a, b = [0, 3, 9, 40, 511, 2047], [5, 1, 7, 2, 100, 1]
    ya = R.rope(x, a)
    assert torch.allclose(ya.norm(dim=-1), x.norm(dim=-1), atol=1e-12, rtol=0)
    yab = R.rope(ya, b)
    assert torch.allclose(yab, R.rope(x, [u + v for u, v in zip(a, b)]), atol=1e-10, rtol=0)
    assert torch.allclose(R.rope(ya, a, inverse=True), x, atol=1e-12, rtol=0)


def test_scores_depend_only_on_position_difference():
    q, k = _x(T=1, H=1, D=32, seed=1), _x(T=1, H=1, D=32, seed=2)
    base = [(R.rope(q, [p + 7]) * R.rope(k, [p])).sum() for p in (0, 5, 100, 3000)]
    for v in base[1:]:
        assert abs(float(v - base[0])) < 1e-9


def test_interleaved_is_a_permutation_of_rotate_half():
    x = _x(T=4, H=2, D=8)
    pos = [0, 2, 5, 11]
    perm = [0, 2, 4, 6, 1, 3, 5, 7]  # interleaved dim j -> rotate-half dim
    inv = np.argsort(perm)
    yi = R.rope(x, pos, interleaved=True)
    yh = R.rope(x[..., perm], pos)
    assert torch.allclose(yi, yh[..., inv], atol=1e-12, rtol=0)
    # and it is the interleaved helper the packed-equals-pairwise pins use
    assert torch.allclose(yi, interleaved_helper(x, pos), atol=1e-12, rtol=0)


def test_packed_rope_uses_aligned_positions():
    """A pack (p=3, responses 2 and 2): the second response's tokens are
    rotated exactly like the first response's (same positions 3, 4)."""
    P, Rl = descriptors([(0, 0, 3, (2, 2))])
    pos, _, _, _ = oracle.positions(P, Rl, 1, 8)
    assert pos[0].tolist() == [0, 1, 2, 3, 4, 3, 4, 0]
    x = _x(T=8, H=1, D=8)[None]
    x[0, 5:7] = x[0, 3:5]
    y = R.packed_rope(x, pos)
    assert torch.equal(y[0, 5:7], y[0, 3:5])
    assert torch.equal(y[0, 7], x[0, 7])  # pad: identity
