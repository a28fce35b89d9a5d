"""Pins of the oracle's lightning-indexer scores and top-k selection."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import indexer as oi
from oracle import quant as oq

RNG = np.random.default_rng(5)


def test_visible_prefix_needs_the_whole_group():
    # entry i is usable once its last token (i+1)*m - 1 exists
    assert [oi.visible_count(t, 64, 4) for t in range(9)] == [0, 0, 0, 1, 1, 1, 1, 2, 2]
    assert oi.visible_count(1_048_575, 262_144, 4) == 262_144
    assert oi.visible_count(1_048_575, 8_192, 128) == 8_192
    assert oi.visible_count(10_000, 50, 4) == 50


def test_single_head_unit_weight_is_relu_of_dot():
    q = RNG.standard_normal((1, 32))
    k = RNG.standard_normal((40, 32))
    s = oi.index_scores(q, np.ones(1), k, 40)
    ref = torch.relu(torch.from_numpy(k) @ torch.from_numpy(q[0])).numpy()
    np.testing.assert_allclose(s, ref, rtol=1e-13)


def test_relu_identities_pin_sign_and_weighting():
    # relu(x) + relu(-x) = |x| and relu(x) - relu(-x) = x: the second collapses all heads into one
    # weighted query, which a dropped ReLU or a sign slip would break.
    H, D, N = 6, 32, 50
    q = RNG.standard_normal((H, D))
    w = RNG.standard_normal(H)
    k = RNG.standard_normal((N, D))
    sp = oi.index_scores(q, w, k, N)
    sm = oi.index_scores(-q, w, k, N)
    np.testing.assert_allclose(sp - sm, k @ (w @ q), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(sp + sm, np.abs(k @ q.T) @ w, rtol=1e-10, atol=1e-10)


def test_invisible_entries_score_minus_inf():
    q = RNG.standard_normal((2, 8))
    k = RNG.standard_normal((10, 8))
    s = oi.index_scores(q, np.ones(2), k, 6)
    assert np.isneginf(s[6:]).all() and np.isfinite(s[:6]).all()


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_quantised_scores_are_exact(fmt):
    # Decoded fp8/fp4 values are dyadic rationals: exact rational arithmetic gives the true score.
    H, D, N = 4, 128, 6
    q = RNG.standard_normal((H, D))
    w = RNG.uniform(0, 1, H)
    k = RNG.standard_normal((N, D))
    qt = oi.quantize_query(q, fmt)
    codes, sc = oi.quantize_keys(k, fmt)
    kt = oi.dequantize_keys(codes, sc, fmt)
    s = oi.index_scores(qt, w, kt, N)
    for i in range(N):
        tot = Fraction(0)
        for h in range(H):
            dot = sum(Fraction(float(qt[h, e])) * Fraction(float(kt[i, e])) for e in range(D))
            tot += Fraction(float(w[h])) * max(dot, Fraction(0))
        assert abs(s[i] - float(tot)) <= 1e-12 * max(1.0, abs(float(tot)))


def test_quantize_query_uses_the_key_rule():
    q = RNG.standard_normal((4, 128))
    np.testing.assert_array_equal(oi.quantize_query(q, "f32"), q)
    c, s = oq.quantize_fp8_rows(q)
    np.testing.assert_array_equal(oi.quantize_query(q, "fp8"), oq.dequantize_fp8_rows(c, s))
    c, s = oq.quantize_mxfp4(q)
    np.testing.assert_array_equal(oi.quantize_query(q, "mxfp4"), oq.dequantize_mxfp4(c, s))


def test_topk_matches_stable_library_sort_and_torch():
    s = RNG.standard_normal(500)
    sel = oi.topk(s, 32, 400)
    ref = np.sort(np.argsort(-s[:400], kind="stable")[:32])
    np.testing.assert_array_equal(sel, ref)
    tv, ti = torch.topk(torch.from_numpy(s[:400]), 32)
    np.testing.assert_array_equal(sel, np.sort(ti.numpy()))
    np.testing.assert_array_equal(oi.topk_fast(s, 32, 400), sel)


def test_topk_ties_go_to_lower_index_and_padding():
    s = np.array([1.0, 3.0, 3.0, 2.0, 3.0, 0.0])
    np.testing.assert_array_equal(oi.topk(s, 2, 6), [1, 2])
    np.testing.assert_array_equal(oi.topk(s, 3, 6), [1, 2, 4])
    np.testing.assert_array_equal(oi.topk(s, 8, 6), [0, 1, 2, 3, 4, 5, -1, -1])
    np.testing.assert_array_equal(oi.topk(s, 4, 0), [-1, -1, -1, -1])
    np.testing.assert_array_equal(oi.topk_fast(s, 3, 6), [1, 2, 4])
    s2 = np.zeros(50)
    np.testing.assert_array_equal(oi.topk_fast(s2, 5, 50), [0, 1, 2, 3, 4])


# ---- indexer keys produced by compression ----------------------------------------------------
def test_compressed_keys_pool_like_the_kv_compressor():
    # Special case -> library: zero logits and bias make every weight equal, so each key is the
    # plain mean of its tokens (torch's avg_pool1d, independently); without overlap the groups
    # are the pooling windows.
    import torch
    rng = np.random.default_rng(5)
    T, D, m = 48, 32, 4
    x = rng.standard_normal((T, D))
    keys, lo = oi.compress_keys(x, np.zeros((T, D)), np.zeros((m, D)), m, 0)
    ref = torch.nn.functional.avg_pool1d(torch.from_numpy(x.T[None]), m).numpy()[0].T
    assert lo == 0 and keys.shape == (T // m, D)
    np.testing.assert_allclose(keys, ref, rtol=0, atol=1e-12)


def test_compressed_keys_of_a_constant_stream_are_the_constant():
    # the pooling weights sum to one in every channel, whatever the logits: a constant token row
    # compresses to itself (with overlap too, including entry 0 with no previous group)
    rng = np.random.default_rng(6)
    T, D, m = 40, 16, 4
    v = rng.standard_normal(D)
    keys, _ = oi.compress_keys(np.tile(v, (T, 1)), rng.standard_normal((T, D)),
                               0.3 * rng.standard_normal((2 * m, D)), m, 1)
    np.testing.assert_allclose(keys, np.tile(v, (T // m, 1)), rtol=0, atol=1e-12)


def test_compressed_keys_are_not_normalised():
    # scaling the stream scales the keys (an RMSNorm would undo it)
    rng = np.random.default_rng(8)
    T, D, m = 32, 16, 4
    x, z, b = rng.standard_normal((T, D)), rng.standard_normal((T, D)), rng.standard_normal((2 * m, D))
    k1, _ = oi.compress_keys(x, z, b, m, 1)
    k3, _ = oi.compress_keys(3.0 * x, z, b, m, 1)
    np.testing.assert_allclose(k3, 3.0 * k1, rtol=1e-12, atol=1e-12)
