"""Pins of the oracle's compressor, RMSNorm and RoPE against facts outside the oracle."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import compress as oc

RNG = np.random.default_rng(7)


def _golden():
    rows = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, val, tol = line.split()[:3]
            rows.setdefault(key, []).append((float(val), float(tol)))
    return rows


def test_entry_counts_match_page_figures():
    g = _golden()
    T = 1 << 20
    lo, hi = oc.entry_range(0, T, 128, 0)
    for val, tol in g["hca_entries_at_1m"]:
        assert abs((hi - lo) - val) <= tol * val
    lo, hi = oc.entry_range(0, T, 4, 1)
    for val, tol in g["csa_entries_at_max"]:
        assert abs((hi - lo) - val) <= tol * val
    assert (hi - lo) == T // 4


@pytest.mark.parametrize("m,overlap", [(4, 1), (4, 0), (128, 0), (8, 1)])
def test_zero_logits_give_average_pooling(m, overlap):
    # Special case -> library: with z = bias = 0 every weight is equal, so each entry is the plain
    # mean of its tokens; torch's avg_pool1d computes that independently.
    T, d = 16 * m, 24
    c = RNG.standard_normal((T, d))
    z = np.zeros((T, d))
    bias = np.zeros(((1 + overlap) * m, d))
    lo, hi = oc.entry_range(0, T, m, overlap)
    pooled = np.stack([oc.pool_entry(c, z, bias, i, m, overlap)[0] for i in range(lo, hi)])
    x = torch.from_numpy(c.T[None])
    if overlap:
        ref = torch.nn.functional.avg_pool1d(x, 2 * m, m, padding=m, count_include_pad=False)[0].T
        ref = ref[: hi - lo]
    else:
        ref = torch.nn.functional.avg_pool1d(x, m, m)[0].T
    np.testing.assert_allclose(pooled, ref.numpy(), rtol=0, atol=1e-12)


def test_softmax_weights_are_a_convex_combination():
    m, o, d = 4, 1, 32
    T = 40
    c = RNG.standard_normal((T, d))
    z = RNG.standard_normal((T, d)) * 3
    bias = RNG.standard_normal((8, d))
    for i in range(T // m):
        p, alpha = oc.pool_entry(c, z, bias, i, m, o)
        np.testing.assert_allclose(alpha.sum(0), 1.0, atol=1e-12)
        assert (alpha > 0).all()
        toks, _ = oc.entry_tokens(i, m, o)
        assert (p <= c[toks].max(0) + 1e-12).all() and (p >= c[toks].min(0) - 1e-12).all()


def test_constant_group_compresses_to_itself():
    m, o, d = 4, 1, 16
    c = np.repeat(RNG.standard_normal((1, d)), 32, axis=0)
    z = RNG.standard_normal((32, d))
    bias = RNG.standard_normal((8, d))
    for i in range(8):       # includes entry 0, which has no previous group
        p, _ = oc.pool_entry(c, z, bias, i, m, o)
        np.testing.assert_allclose(p, c[0], atol=1e-12)


@pytest.mark.parametrize("slot", range(8))
def test_bias_slot_layout_with_overlap(slot):
    # A dominant bias on one slot selects one token: slots 0..3 are the previous group and 4..7
    # the own group, in token order.  Entry 0 has no previous group: its own slots tie.
    m, o, d, T = 4, 1, 8, 32
    c = RNG.standard_normal((T, d))
    z = np.zeros((T, d))
    bias = np.zeros((8, d))
    bias[slot] = 80.0
    for i in range(T // m):
        p, _ = oc.pool_entry(c, z, bias, i, m, o)
        if i == 0 and slot < m:
            np.testing.assert_allclose(p, c[0:m].mean(0), atol=1e-12)
        else:
            np.testing.assert_allclose(p, c[(i - 1) * m + slot], atol=1e-12)


def test_hca_slot_layout_and_ratio_one():
    m, d = 128, 8
    c = RNG.standard_normal((4 * m, d))
    z = np.zeros_like(c)
    bias = np.zeros((m, d))
    bias[77] = 80.0
    for i in range(4):
        p, _ = oc.pool_entry(c, z, bias, i, m, 0)
        np.testing.assert_allclose(p, c[i * m + 77], atol=1e-12)
    # m = 1 without overlap: every token is its own entry
    zz = RNG.standard_normal((16, d))
    e = np.stack([oc.pool_entry(c[:16], zz, np.zeros((1, d)), i, 1, 0)[0] for i in range(16)])
    np.testing.assert_allclose(e, c[:16], atol=1e-12)


def test_large_logit_limit_picks_token():
    m, o, d = 4, 1, 4
    c = RNG.standard_normal((16, d))
    z = RNG.standard_normal((16, d))
    z[9, 2] = 200.0
    p, _ = oc.pool_entry(c, z, np.zeros((8, d)), 2, m, o)   # entry 2 spans tokens 4..11
    assert abs(p[2] - c[9, 2]) < 1e-12


def test_rmsnorm_matches_torch_and_invariants():
    x = RNG.standard_normal((5, 64)) * 3
    w = RNG.standard_normal(64)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(w), eps=1e-6)
    np.testing.assert_allclose(oc.rms_norm(x, w, 1e-6), ref.numpy(), rtol=1e-12, atol=1e-12)
    y = oc.rms_norm(x, None, 0.0)
    np.testing.assert_allclose(np.sqrt((y * y).mean(-1)), 1.0, atol=1e-12)
    np.testing.assert_allclose(oc.rms_norm(7.5 * x, None, 0.0), y, atol=1e-12)


@pytest.mark.parametrize("rope_dim,D", [(16, 64), (64, 512)])
def test_rope_matches_gptj_interleaved_rotary(rope_dim, D):
    # Library pin: GPT-J's rotary embedding rotates interleaved pairs with base 10000.
    from transformers.models.gptj import modeling_gptj as gptj
    npos = 300
    x = RNG.standard_normal((npos, D))
    ours = oc.rope(x, np.arange(npos), rope_dim)
    sincos = gptj.create_sinusoidal_positions(npos, rope_dim)            # [npos, rope_dim]
    sin, cos = sincos[:, : rope_dim // 2], sincos[:, rope_dim // 2:]
    t = torch.from_numpy(x[:, D - rope_dim:]).float()[None, :, None, :]    # [1, seq, 1, r]
    ref = gptj.apply_rotary_pos_emb(t, sin[None], cos[None])[0, :, 0].double().numpy()
    np.testing.assert_allclose(ours[:, D - rope_dim:], ref, atol=2e-4)
    np.testing.assert_array_equal(ours[:, : D - rope_dim], x[:, : D - rope_dim])


def test_rope_invariants_and_complex_form_at_large_positions():
    r, D = 64, 128
    x = RNG.standard_normal((D,))
    y = RNG.standard_normal((D,))
    np.testing.assert_allclose(oc.rope(x, 0, r), x, atol=0)
    for pos in (1, 1000, 1048575):
        rx = oc.rope(x, pos, r)
        # pair norms preserved
        a0 = x[D - r:].reshape(-1, 2)
        a1 = rx[D - r:].reshape(-1, 2)
        np.testing.assert_allclose(np.hypot(*a1.T), np.hypot(*a0.T), rtol=1e-12)
        # independent formulation: each pair is a complex number multiplied by exp(i*phi)
        zc = a0[:, 0] + 1j * a0[:, 1]
        theta = np.array([10000.0 ** (-(2 * u) / r) for u in range(r // 2)])
        zr = zc * np.exp(1j * pos * theta)
        np.testing.assert_allclose(a1[:, 0], zr.real, atol=1e-9)
        np.testing.assert_allclose(a1[:, 1], zr.imag, atol=1e-9)
    # relative positions: <R(a)x, R(b)y> depends only on b - a
    for a, b, dlt in ((3, 10, 1000), (0, 5, 1048000)):
        v1 = oc.rope(x, a, r) @ oc.rope(y, b, r)
        v2 = oc.rope(x, a + dlt, r) @ oc.rope(y, b + dlt, r)
        assert abs(v1 - v2) < 1e-8 * (1 + abs(v1))


def test_compress_places_entries_at_their_group_start_and_chunks_agree():
    # A chunk with an m-row halo must reproduce the entries of the whole-sequence pass.
    m, o, d, r = 4, 1, 32, 8
    T = 64
    c = RNG.standard_normal((T, d))
    z = RNG.standard_normal((T, d))
    bias = RNG.standard_normal((8, d)) * 0.1
    full, lo, _ = oc.compress(c, z, bias, m, o, r)
    assert lo == 0 and full.shape[0] == T // m
    pos0 = 32
    part, lo2, _ = oc.compress(c[pos0 - m:], z[pos0 - m:], bias, m, o, r, pos_first=pos0 - m)
    assert lo2 == pos0 // m
    np.testing.assert_allclose(part, full[lo2:], atol=1e-12)
    # the rotation uses the entry position i*m: undoing it gives the normalised pooled value
    pooled = np.stack([oc.pool_entry(c, z, bias, i, m, o)[0] for i in range(T // m)])
    for i in (1, 5, 15):
        back = oc.rope(full[i], -i * m, r)
        np.testing.assert_allclose(back, oc.rms_norm(pooled[i]), atol=1e-12)


def test_window_rows_are_normalised_and_rotated_per_token():
    d, r = 64, 16
    c = RNG.standard_normal((10, d)) * 5
    rows = oc.window_rows(c, r, pos_first=100)
    np.testing.assert_allclose(np.sqrt((rows ** 2).mean(-1)), 1.0, atol=1e-5)
    back = oc.rope(rows[3], -103, r)
    np.testing.assert_allclose(back, c[3] / math.sqrt((c[3] ** 2).mean() + 1e-6), atol=1e-12)
