"""Pins of the oracle's core attention and of the whole CSA pass on the tiny workload."""
import math

import numpy as np
import torch

from compressed_sparse_attention_03_amd import inputs as gen
from oracle import attention as oa
from oracle import compress as oc
from oracle import pipeline as op

RNG = np.random.default_rng(3)


def _sdpa(q_hat, X, mask=None):
    # library: scaled_dot_product_attention in float64 with the single KV head expanded
    qh = torch.from_numpy(q_hat)[None, :, None, :]                  # [1, H, 1, D]
    kv = torch.from_numpy(X)[None, None].expand(1, q_hat.shape[0], -1, -1)
    return torch.nn.functional.scaled_dot_product_attention(qh, kv, kv)[0, :, 0].numpy()


def test_mqa_matches_sdpa_and_logsumexp():
    H, D, n = 8, 64, 37
    q = RNG.standard_normal((H, D))
    X = RNG.standard_normal((n, D))
    o, lse = oa.mqa(q, X, 1 / math.sqrt(D))
    np.testing.assert_allclose(o, _sdpa(q, X), atol=1e-12)
    ref = torch.logsumexp(torch.from_numpy(q @ X.T / math.sqrt(D)), dim=1).numpy()
    np.testing.assert_allclose(lse, ref, atol=1e-12)


def test_special_cases():
    H, D = 4, 32
    X = RNG.standard_normal((9, D))
    o, _ = oa.mqa(np.zeros((H, D)), X, 0.3)                          # q = 0 -> mean of the rows
    np.testing.assert_allclose(o, np.repeat(X.mean(0, keepdims=True), H, 0), atol=1e-12)
    q = RNG.standard_normal((H, D))
    o, lse = oa.mqa(q, X[:1], 0.3)                                    # one row -> that row
    np.testing.assert_allclose(o, np.repeat(X[:1], H, 0), atol=1e-12)
    np.testing.assert_allclose(lse, q @ X[0] * 0.3, atol=1e-12)


def test_window_positions():
    assert oa.window_positions(0, 128) == [0]
    assert oa.window_positions(5, 3) == [3, 4, 5]
    assert len(oa.window_positions(1_048_575, 128)) == 128


def test_selection_order_and_padding_do_not_matter():
    H, D, N, W = 4, 64, 40, 8
    q = RNG.standard_normal((H, D))
    ent = RNG.standard_normal((N, D))
    win = RNG.standard_normal((W, D))
    t = 1000
    sel = np.array([3, 17, 5, 30, 1])
    a = oa.csa_attend(q, ent, sel, win, t - W + 1, t, W, 16)
    b = oa.csa_attend(q, ent, np.concatenate([sel[::-1], [-1, -1]]), win, t - W + 1, t, W, 16)
    np.testing.assert_allclose(a[0], b[0], atol=1e-12)
    np.testing.assert_allclose(a[1], b[1], atol=1e-12)


def test_hca_equals_csa_with_every_visible_entry():
    H, D, N, W = 4, 64, 30, 8
    q = RNG.standard_normal((H, D))
    ent = RNG.standard_normal((N, D))
    win = RNG.standard_normal((W, D))
    a = oa.hca_attend(q, ent, 25, win, 100 - W + 1, 100, W, 16)
    b = oa.csa_attend(q, ent, np.arange(25), win, 100 - W + 1, 100, W, 16)
    np.testing.assert_allclose(a[0], b[0], atol=0)


def _tiny(topk=None, window=None):
    w = gen.TINY
    x = gen.tiny_inputs(w)
    f = lambda a: gen.bf16_bits_to_f32(a).astype(np.float64)
    return w, x, op.csa_forward(f(x["c"][0]), f(x["z"][0]), f(x["bias"]), f(x["q"][0]), x["q_idx"][0],
                                x["w_idx"][0], x["k_idx"][0], m=w.m, overlap=w.overlap,
                                rope_dim=w.rope_dim, topk=topk or w.topk, window=window or w.window,
                                key_format="f32")


def test_full_selection_and_full_window_reduce_to_dense_attention():
    # With top-k covering every entry and the window covering the sequence, CSA is dense MQA over
    # the visible compressed entries plus every past token row (checked with the library's SDPA).
    w, x, out = _tiny(topk=64, window=256)
    ent, rows = out["entries"], out["win_rows"]
    f = lambda a: gen.bf16_bits_to_f32(a).astype(np.float64)
    q = f(x["q"][0])
    for t in (0, 2, 3, 50, 137, 255):
        nv = (t + 1) // 4
        X = np.concatenate([ent[:nv], rows[: t + 1]], 0)
        q_hat = oc.rope(oc.rms_norm(q[t]), t, w.rope_dim)
        np.testing.assert_allclose(out["o"][t], _sdpa(q_hat, X), atol=1e-12)


def test_tiny_pipeline_early_queries_see_only_the_window():
    w, x, out = _tiny()
    for t in (0, 1, 2):
        assert (out["topk"][t] == -1).all()
    assert (out["topk"][3][1:] == -1).all() and out["topk"][3][0] == 0
    for t in (10, 40, 62):
        nv = (t + 1) // 4
        assert (out["topk"][t] >= 0).sum() == min(16, nv)
    for t in (100, 255):
        assert (out["topk"][t] >= 0).sum() == 16
        assert np.isfinite(out["o"][t]).all()
    # query 0 attends to its own row only
    rows = out["win_rows"]
    np.testing.assert_allclose(out["o"][0], np.repeat(rows[:1], w.H, 0), atol=1e-12)
