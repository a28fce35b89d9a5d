"""End-to-end oracle passes: compress -> index -> top-k -> attend (CSA) and compress -> attend (HCA).

[EXPLAINER] CSA walk-through: compressor, lightning indexer, top-k selector, then core attention
over the picked entries plus a sliding window.  [SUMMARY] section 2.3: CSA compresses every m
tokens and attends to the top-k entries chosen by the lightning indexer; HCA compresses every
m' tokens and attends densely.  Test infrastructure only.
"""
from __future__ import annotations

import math

import numpy as np

from . import attention, compress, indexer


def csa_forward(c, z, bias, q, q_idx, w_idx, k_idx, *, m, overlap, rope_dim, topk, window,
                key_format="f32", norm_w=None, q_norm_w=None, eps=1e-6, rope_base=10000.0,
                queries=None):
    """One CSA layer over a sequence starting at position 0, for every causal query token.

    c, z [T, d]; bias [(1+overlap)m, d]; q [T, H, d]; q_idx [T, H_I, D_I]; w_idx [T, H_I];
    k_idx [N, D_I] (one indexer key per compressed entry, unquantised).
    Returns a dict of every intermediate and the outputs o [T, H, d], lse [T, H].
    """
    T, d = c.shape
    entries, lo, pooled = compress.compress(c, z, bias, m, overlap, rope_dim, norm_w, eps, rope_base)
    assert lo == 0
    N = entries.shape[0]
    rows = compress.window_rows(c, rope_dim, norm_w, eps, rope_base)
    codes, scales = indexer.quantize_keys(k_idx[:N], key_format)
    k_tilde = indexer.dequantize_keys(codes, scales, key_format)
    H = q.shape[1]
    queries = range(T) if queries is None else queries
    out = {"entries": entries, "pooled": pooled, "win_rows": rows, "k_tilde": k_tilde,
           "scores": {}, "topk": {}, "o": np.zeros((T, H, d)), "lse": np.zeros((T, H))}
    for t in queries:
        nv = indexer.visible_count(t, N, m)
        qt = indexer.quantize_query(q_idx[t], key_format)
        s = indexer.index_scores(qt, w_idx[t], k_tilde, nv)
        sel = indexer.topk(s, topk, nv)
        o, lse = attention.csa_attend(q[t], entries, sel, rows, 0, t, window, rope_dim,
                                      1.0 / math.sqrt(d), q_norm_w, eps, rope_base)
        out["scores"][t], out["topk"][t] = s, sel
        out["o"][t], out["lse"][t] = o, lse
    return out
