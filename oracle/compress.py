"""Oracle step 1: the KV compressor (softmax pooling per channel), RMSNorm and partial RoPE.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np


def entry_tokens(i: int, m: int, overlap: int):
    """Token positions pooled into compressed entry ``i`` and the bias slot of each.

    [EXPLAINER] CSA walk-through: every m = 4 raw tokens become one compressed entry.
    [RABBIT] CSA paragraph: an entry's pooling also covers the four tokens of the group before it.
    [EXPLAINER] HCA walk-through: HCA pools disjoint runs of m' = 128 tokens.

    Reading: with overlap the entry spans its own group [i*m, (i+1)*m) and the previous group
    [(i-1)*m, i*m); bias slots 0..m-1 belong to the previous group and m..2m-1 to the own group,
    in ascending token order.  Entry 0 has no previous group: its missing slots are left out of
    the softmax (so a constant group still compresses to itself).
    """
    if overlap:
        first = (i - 1) * m
        toks = [t for t in range(first, (i + 1) * m) if t >= 0]
        slots = [t - first for t in toks]
    else:
        toks = list(range(i * m, (i + 1) * m))
        slots = [t - i * m for t in toks]
    return toks, slots


def pool_entry(c: np.ndarray, z: np.ndarray, bias: np.ndarray, i: int, m: int, overlap: int,
               pos_first: int = 0):
    """Softmax-weighted pooling of one entry, channel by channel.

    [EXPLAINER] CSA walk-through: the group's tokens are combined with learned softmax weights.
    [DEVTO] "Two Compression Strategies": runs of consecutive tokens are merged by pooling with
    softmax weights.  [RABBIT] HCA paragraph: the averages are weighted, and the weights change
    from one channel of the representation to another (so the softmax is taken per channel).

    Reading: the weight logit of token t in channel j is z[t, j] + bias[slot(t), j].

    ``c``/``z`` hold rows for positions pos_first, pos_first+1, ...  Returns (p, alpha) with
    p[j] = sum_t alpha[t, j] * c[t, j] and alpha the per-channel softmax over the entry's tokens.
    """
    toks, slots = entry_tokens(i, m, overlap)
    rows = np.array([t - pos_first for t in toks])
    assert rows.min() >= 0 and rows.max() < c.shape[0], "entry tokens not all present"
    logits = z[rows].astype(np.float64) + bias[np.array(slots)].astype(np.float64)
    logits = logits - logits.max(axis=0, keepdims=True)
    e = np.exp(logits)
    alpha = e / e.sum(axis=0, keepdims=True)
    p = (alpha * c[rows].astype(np.float64)).sum(axis=0)
    return p, alpha


def rms_norm(x: np.ndarray, weight: np.ndarray | None = None, eps: float = 1e-6) -> np.ndarray:
    """RMSNorm over the last axis.

    [SUMMARY] section 2.3, "Other details": both the query heads and the compressed KV entries
    are RMS-normalised just before core attention.  [DEVTO]: query and KV normalisation.
    Reading: eps = 1e-6; weight defaults to ones (no trained weights exist here).
    """
    x = x.astype(np.float64)
    r = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    if weight is not None:
        r = r * weight.astype(np.float64)
    return r


def rope(x: np.ndarray, pos, rope_dim: int, base: float = 10000.0) -> np.ndarray:
    """Partial rotary position embedding on the last ``rope_dim`` channels.

    [DEVTO] "Two Compression Strategies": both CSA and HCA use partial RoPE.

    Reading (parity unpinned by the pages; pinned to GPT-J's interleaved rotary form): pair u
    covers channels a = D - r + 2u and a + 1, it turns by angle pos * base**(-2u/r), and
    (x_a, x_b) -> (x_a cos - x_b sin, x_a sin + x_b cos).  Angles are formed in float64.
    ``pos`` is a scalar or an array broadcasting against x[..., 0].
    """
    x = np.array(x, dtype=np.float64, copy=True)
    D = x.shape[-1]
    if rope_dim == 0:
        return x
    u = np.arange(rope_dim // 2, dtype=np.float64)
    theta = base ** (-2.0 * u / rope_dim)
    phi = np.asarray(pos, dtype=np.float64)[..., None] * theta
    cos, sin = np.cos(phi), np.sin(phi)
    a = x[..., D - rope_dim::2].copy()
    b = x[..., D - rope_dim + 1::2].copy()
    x[..., D - rope_dim::2] = a * cos - b * sin
    x[..., D - rope_dim + 1::2] = a * sin + b * cos
    return x


def entry_range(pos_first: int, n_rows: int, m: int, overlap: int):
    """Entries whose tokens all lie in the given rows (or before position 0).

    [RABBIT] sliding-window paragraph: tokens of an unfinished group are not in any entry yet,
    so an entry exists only once its whole group is present.
    """
    assert pos_first % m == 0
    lo = pos_first // m + (1 if (overlap and pos_first > 0) else 0)
    hi = (pos_first + n_rows) // m
    return lo, max(lo, hi)


def compress(c, z, bias, m, overlap, rope_dim, norm_w=None, eps=1e-6, rope_base=10000.0,
             pos_first=0):
    """Compressed KV entries for every complete entry in the rows: pool -> RMSNorm -> RoPE.

    Each entry is placed at the position of the first token of its own group (i * m).
    Returns (entries [n, d] float64, first entry index, pooled-before-norm [n, d]).
    """
    lo, hi = entry_range(pos_first, c.shape[0], m, overlap)
    pooled = np.stack([pool_entry(c, z, bias, i, m, overlap, pos_first)[0] for i in range(lo, hi)]) \
        if hi > lo else np.zeros((0, c.shape[1]))
    normed = rms_norm(pooled, norm_w, eps)
    pos = np.arange(lo, hi) * m
    return rope(normed, pos, rope_dim, rope_base), lo, pooled


def window_rows(c, rope_dim, norm_w=None, eps=1e-6, rope_base=10000.0, pos_first=0):
    """Per-token rows for the sliding window: RMSNorm then RoPE at the token's own position.

    [RABBIT] sliding-window paragraph: the newest 128 tokens are also kept uncompressed, each as
    its own row.  Reading: these rows get the same normalisation and rotation as the
    compressed entries, so every key in the joint softmax sits on one scale.
    """
    pos = pos_first + np.arange(c.shape[0])
    return rope(rms_norm(c, norm_w, eps), pos, rope_dim, rope_base)
