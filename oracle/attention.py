"""Oracle step 4: shared-KV multi-query core attention over (selected entries + sliding window).

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import math

import numpy as np

from .compress import rms_norm, rope


def prepare_query(q: np.ndarray, t: int, rope_dim: int, norm_w=None, eps=1e-6, rope_base=10000.0):
    """Query heads right before core attention: per-head RMSNorm, then partial RoPE at t.

    [SUMMARY] section 2.3, "Other details": RMSNorm on the query heads before core attention.
    [DEVTO]: partial RoPE.  q is [H, D].
    """
    return rope(rms_norm(q, norm_w, eps), t, rope_dim, rope_base)


def window_positions(t: int, window: int):
    """Positions seen raw through the sliding window: max(0, t-W+1) .. t (always contains t).

    [RABBIT] sliding-window paragraph: the newest 128 tokens are also kept as their own rows, so
    a token whose group is not yet complete can still be seen right away.
    """
    return list(range(max(0, t - window + 1), t + 1))


def mqa(q_hat: np.ndarray, X: np.ndarray, scale: float):
    """Softmax attention of every query head over the same rows X (shared KV: K = V = X).

    [SUMMARY] section 2.3, "Shared KV and output projection": shared-KV multi-query attention.
    [EXPLAINER] HCA walk-through: HCA uses ordinary multi-query attention arithmetic.
    Reading: K and V are the same prepared row; logits are <q_h, x> * scale; one softmax per head
    over all rows (max-subtracted); lse is the natural-log normaliser.
    Returns (o [H, D], lse [H]).
    """
    logits = (q_hat @ X.T) * scale                      # [H, n]
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    ssum = e.sum(axis=1, keepdims=True)
    o = (e / ssum) @ X
    lse = (mx + np.log(ssum))[:, 0]
    return o, lse


def gather_rows(entries, sel, win_rows, win_pos0: int, t: int, window: int):
    """X(t) = selected compressed entries followed by the window rows (one joint softmax).

    [EXPLAINER] CSA walk-through: every query head's attention covers the selected entries
    together with a window of the newest tokens.  Reading: one joint softmax over the union (equivalently two
    branches merged by their log-sum-exp); a token may be seen both raw and inside an entry.
    """
    sel = [int(i) for i in sel if i >= 0]
    wpos = window_positions(t, window)
    rows_e = np.asarray(entries, dtype=np.float64)[sel] if sel else np.zeros((0, entries.shape[1]))
    idx = [p - win_pos0 for p in wpos]
    assert min(idx) >= 0 and max(idx) < win_rows.shape[0], "window rows not supplied"
    rows_w = np.asarray(win_rows, dtype=np.float64)[idx]
    return np.concatenate([rows_e, rows_w], axis=0)


def csa_attend(q, entries, topk_idx, win_rows, win_pos0, t, window, rope_dim, scale=None,
               q_norm_w=None, eps=1e-6, rope_base=10000.0):
    """CSA core attention for one query token: q [H, D] raw heads -> (o [H, D], lse [H])."""
    D = q.shape[-1]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    q_hat = prepare_query(q, t, rope_dim, q_norm_w, eps, rope_base)
    X = gather_rows(entries, topk_idx, win_rows, win_pos0, t, window)
    return mqa(q_hat, X, scale)


def hca_attend(q, entries, n_visible, win_rows, win_pos0, t, window, rope_dim, scale=None,
               q_norm_w=None, eps=1e-6, rope_base=10000.0):
    """HCA core attention: dense over every visible compressed entry plus the window.

    [EXPLAINER] HCA walk-through: no selection step -- each query sees every compressed entry,
    together with a short window of the newest raw tokens.
    """
    return csa_attend(q, entries, list(range(n_visible)), win_rows, win_pos0, t, window, rope_dim,
                      scale, q_norm_w, eps, rope_base)
