"""Oracle of the grouped output projection after core attention.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np


def grouped_output_projection(o: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Hidden state from the core-attention head outputs through a grouped projection.

    [SUMMARY] 2.3 "Hybrid Attention with CSA and HCA", shared-KV and output-projection paragraph:
    both attention types map their many head outputs back to the model width through a
    projection split into groups, to cut that cost.

    Reading: the heads are split into G equal groups in head order; group g's head outputs,
    concatenated in head order, are projected by its own weight w[g] (out_features x
    in_features, as a linear layer stores it) to N_g outputs, and the G results are concatenated
    -- a block-diagonal linear map costing 1/G of a dense one.

    o: [M, H*D] (tokens x concatenated heads); w: [G, N_g, H*D/G].  Returns y [M, G*N_g].
    """
    o = np.asarray(o, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    G, N_g, K_g = w.shape
    assert o.shape[1] == G * K_g
    return np.concatenate([o[:, g * K_g:(g + 1) * K_g] @ w[g].T for g in range(G)], axis=1)
