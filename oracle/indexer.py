"""Oracle steps 2b and 3: lightning-indexer scores and per-query top-k selection.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from . import quant


def visible_count(t: int, n_entries: int, m: int) -> int:
    """Number of compressed entries a query at position ``t`` may use.

    [EXPLAINER] CSA walk-through: compression comes first and selection second, so only entries
    that already exist can be scored.  Reading: entry i becomes usable once its last token exists, (i+1)*m - 1 <= t, so the
    visible set is the prefix [0, min(n_entries, (t+1) // m)).
    """
    return int(min(n_entries, (t + 1) // m))


def quantize_query(q: np.ndarray, fmt: str) -> np.ndarray:
    """The query as the indexer sees it: quantised by the same rule as the keys, then decoded.

    [DEVTO] "Two Compression Strategies": the indexer runs in low precision (FP4); the decode
    configs use fp8 e4m3 or MXFP4.  Reading: the query of each indexer head is quantised with the
    keys' rule (fp8: one power-of-two scale per head row; MXFP4: one e8m0 scale per 32 values).
    """
    if fmt == "f32":
        return np.asarray(q, dtype=np.float64)
    if fmt == "fp8":
        codes, scales = quant.quantize_fp8_rows(q)
        return quant.dequantize_fp8_rows(codes, scales)
    if fmt == "mxfp4":
        codes, sb = quant.quantize_mxfp4(q)
        return quant.dequantize_mxfp4(codes, sb)
    raise ValueError(fmt)


def quantize_keys(k: np.ndarray, fmt: str):
    """Keys in storage form: (codes, scales) for fp8/MXFP4; the fp32 keys themselves otherwise."""
    if fmt == "fp8":
        return quant.quantize_fp8_rows(k)
    if fmt == "mxfp4":
        return quant.quantize_mxfp4(k)
    return np.asarray(k, dtype=np.float64), None


def compress_keys(c_i, z_i, bias_i, m: int, overlap: int, pos_first: int = 0):
    """Indexer keys of the compressed entries, produced by compression of a per-token stream.

    [EXPLAINER] CSA walk-through: the lightning indexer scores compressed blocks, so each entry
    carries its own indexer key; the compressor pools every entry from its group of tokens with
    learned softmax weights.  [RABBIT] indexer paragraph: the indexer's operands are compact (a
    narrower key than the attention rows).

    Reading: a per-token indexer stream c_i [T, D_I] with logits z_i and position bias bias_i
    [(1+overlap) m, D_I] is pooled exactly as the KV compressor pools (same token groups, same
    per-channel softmax), with no RMSNorm and no rotation (the keys are used as they are).
    Returns (keys [n, D_I] float64, first entry index).
    """
    from .compress import entry_range, pool_entry
    lo, hi = entry_range(pos_first, c_i.shape[0], m, overlap)
    keys = np.stack([pool_entry(c_i, z_i, bias_i, i, m, overlap, pos_first)[0] for i in range(lo, hi)]) \
        if hi > lo else np.zeros((0, c_i.shape[1]))
    return keys, lo


def dequantize_keys(codes, scales, fmt: str) -> np.ndarray:
    if fmt == "fp8":
        return quant.dequantize_fp8_rows(codes, scales)
    if fmt == "mxfp4":
        return quant.dequantize_mxfp4(codes, scales)
    return np.asarray(codes, dtype=np.float64)


def index_scores(q_tilde: np.ndarray, w: np.ndarray, k_tilde: np.ndarray, n_visible: int) -> np.ndarray:
    """Relevance of every visible compressed entry to one query token.

    [EXPLAINER] CSA walk-through: the lightning indexer is a lightweight scoring head that rates
    each compressed block for the present query.  [RABBIT] indexer paragraph: it visits all
    compressed entries, so its cost rises with the context length.

    Reading (parity unpinned by the pages): s[i] = sum_h w[h] * max(0, <q_h, k_i>) over the
    indexer heads h, the lightning-indexer form of the predecessor's sparse attention that the
    pages say V4 adapts.  Invisible entries score -inf.

    q_tilde [H_I, D_I], w [H_I], k_tilde [N, D_I] (already decoded), all float64.
    """
    N = k_tilde.shape[0]
    s = np.full(N, -np.inf)
    if n_visible > 0:
        dots = k_tilde[:n_visible] @ q_tilde.T                  # [n, H_I]
        s[:n_visible] = np.maximum(dots, 0.0) @ np.asarray(w, dtype=np.float64)
    return s


def topk(scores: np.ndarray, k: int, n_visible: int) -> np.ndarray:
    """Indices of the min(k, n_visible) best-scoring visible entries, ascending, -1 padded.

    [EXPLAINER] CSA walk-through: the top-k selector keeps only the best entries.
    [RABBIT] indexer paragraph: the top 1,024 entries go on to attention.
    Reading: one set per query token, shared by all query heads; equal scores go to the lower
    index.
    """
    n = min(k, n_visible)
    order = sorted(range(n_visible), key=lambda i: (-scores[i], i))[:n]
    out = np.full(k, -1, dtype=np.int64)
    out[:n] = np.sort(np.asarray(order, dtype=np.int64))
    return out


def topk_fast(scores: np.ndarray, k: int, n_visible: int) -> np.ndarray:
    """Same selection as ``topk`` with a library sort (for long score vectors)."""
    n = min(k, n_visible)
    s = scores[:n_visible]
    order = np.lexsort((np.arange(n_visible), -s))[:n]
    out = np.full(k, -1, dtype=np.int64)
    out[:n] = np.sort(order)
    return out
