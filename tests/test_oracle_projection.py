"""Pins of the oracle's grouped output projection against library routines and its structure."""
import numpy as np
import torch

from oracle import projection as op

RNG = np.random.default_rng(13)


def test_one_group_is_a_dense_linear_layer():
    # special case -> library: with G = 1 the projection is torch's linear layer
    o = RNG.standard_normal((5, 96))
    w = RNG.standard_normal((1, 40, 96))
    ref = torch.nn.functional.linear(torch.from_numpy(o), torch.from_numpy(w[0])).numpy()
    np.testing.assert_allclose(op.grouped_output_projection(o, w), ref, rtol=1e-12, atol=1e-12)


def test_groups_are_a_block_diagonal_linear_layer():
    # the G group weights placed on the diagonal of one dense weight give the same map
    G, N_g, K_g, M = 4, 24, 32, 7
    o = RNG.standard_normal((M, G * K_g))
    w = RNG.standard_normal((G, N_g, K_g))
    dense = torch.block_diag(*[torch.from_numpy(w[g]) for g in range(G)])
    ref = torch.nn.functional.linear(torch.from_numpy(o), dense).numpy()
    np.testing.assert_allclose(op.grouped_output_projection(o, w), ref, rtol=1e-12, atol=1e-12)


def test_a_group_sees_only_its_heads():
    G, N_g, K_g, M = 4, 8, 16, 3
    o = RNG.standard_normal((M, G * K_g))
    w = RNG.standard_normal((G, N_g, K_g))
    y0 = op.grouped_output_projection(o, w)
    o2 = o.copy()
    o2[:, 2 * K_g:3 * K_g] += 1.0                         # change group 2's heads only
    y1 = op.grouped_output_projection(o2, w)
    changed = np.abs(y1 - y0).max(axis=0) > 0
    assert changed[2 * N_g:3 * N_g].all() and not changed[:2 * N_g].any() and not changed[3 * N_g:].any()
