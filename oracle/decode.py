"""Oracle for decode-time cache maintenance: what the caches of one sequence hold once tokens
0..t exist.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .compress import compress, window_rows
from .indexer import quantize_keys


def cache_after(c, z, bias, keys, t: int, *, m: int, overlap: int, rope_dim: int, window: int,
                key_format: str | None = None, norm_w=None, eps: float = 1e-6,
                rope_base: float = 10000.0):
    """Contents of the decode caches once the tokens at positions 0..t exist.

    [EXPLAINER] CSA walk-through: the compressed store gains one entry per m tokens, made by the
    learned softmax pooling (HCA walk-through: per m' = 128 tokens, without overlap).
    [RABBIT] sliding-window paragraph: the most recent tokens are also kept as separate rows,
    and the tokens of an unfinished group belong to no entry yet.
    [RABBIT] indexer paragraph, [DEVTO] "Two Compression Strategies": the indexer reads its keys
    in a low-precision storage format.

    Reading: the caches are a function of the tokens so far and nothing else -- every complete
    entry exactly as the batch compressor makes it, the prepared rows of the last ``window``
    positions, and each entry's indexer key in storage form (quantised once, when the entry is
    written).  The order in which the tokens arrived does not enter.

    c, z: [>= t+1, d] token rows from position 0; keys: [>= n, D_I] the entries' indexer keys.
    Returns a dict: n_entries, entries [n, d], win_pos [w] (positions), win_rows [w, d], and
    key_codes / key_scales when ``key_format`` is given ("fp8", "mxfp4" or "f32").
    """
    n_tok = t + 1
    ent, lo, _ = compress(c[:n_tok], z[:n_tok], bias, m, overlap, rope_dim, norm_w, eps,
                          rope_base, pos_first=0)
    assert lo == 0
    n = ent.shape[0]
    w0 = max(0, t - window + 1)
    win = window_rows(c[w0:n_tok], rope_dim, norm_w, eps, rope_base, pos_first=w0)
    out = dict(n_entries=n, entries=ent, win_pos=np.arange(w0, n_tok), win_rows=win)
    if key_format is not None:
        codes, scales = quantize_keys(np.asarray(keys[:n], dtype=np.float64), key_format)
        out.update(key_codes=codes, key_scales=scales)
    return out
