"""Full-size decode steps exactly as the benchmark runs them: csa_index_topk without scores (the
timed call: fused merge in the last segment workgroup) feeding csa_attend, at the 32K, 128K and 1M
configurations.  The GPU's selection is held to the oracle's scores (exact sets up to near-ties
within 1e-3 of the k-th score, planted entries always kept), and the GPU's attention over that
selection to the oracle's attention over the same selection (the step's end-to-end output)."""
import math

import numpy as np
import pytest

from compressed_sparse_attention_03_amd import inputs as gen
from compressed_sparse_attention_03_amd import ops
from oracle import attention as oa
from oracle import indexer as oi
from helpers import assert_close, assert_topk, dev, dev_bf16, f64, host_f64, say

pytestmark = pytest.mark.gpu


def _oracle_keys(k_bf16_seq: np.ndarray, fmt: str, chunk=32768):
    out = np.empty(k_bf16_seq.shape, dtype=np.float64)
    for i in range(0, k_bf16_seq.shape[0], chunk):
        codes, sc = oi.quantize_keys(f64(k_bf16_seq[i:i + chunk]), fmt)
        out[i:i + chunk] = oi.dequantize_keys(codes, sc, fmt)
    return out


def _chain(w, n_seq):
    x = gen.decode_inputs(w, 0, n_seq)
    say(f"case: decode chain {w.name} sequences 0..{n_seq - 1}")
    codes, scales = ops.csa_quantize_keys(dev_bf16(x["k_idx"]), w.key_format)
    t = dev(x["t"])
    sel, sc = ops.csa_index_topk(dev_bf16(x["q_idx"]), dev(x["w_idx"]), codes, scales, key_format=w.key_format,
                                 n_entries=dev(x["n_entries"]), q_pos0=t, m=w.m, topk=w.topk)
    assert sc is None
    out, lse = ops.csa_attend(dev_bf16(x["q"]), dev_bf16(x["entries"]), sel, dev_bf16(x["win_rows"]),
                              dev(x["win_pos0"]), t, rope_dim=w.rope_dim, window=w.window, lse=True)
    sel = sel.cpu().numpy()
    out, lse = host_f64(out), host_f64(lse)
    planted = gen.planted_indices(w) if w.n_planted else None
    ref_o, ref_l = [], []
    for b in range(n_seq):
        tb = int(x["t"][b])
        nv = oi.visible_count(tb, int(x["n_entries"][b]), w.m)
        kt = _oracle_keys(x["k_idx"][b, :nv], w.key_format)
        qt = oi.quantize_query(f64(x["q_idx"][b, 0]), w.key_format)
        s = oi.index_scores(qt, x["w_idx"][b, 0].astype(np.float64), kt, nv)
        assert_topk(sel[b, 0], s, w.topk, nv, f"topk[{b}]")
        if planted is not None:
            assert set(planted[b].tolist()) <= set(sel[b, 0].tolist()), f"planted entry missed in sequence {b}"
        rows = sel[b, 0][sel[b, 0] >= 0]
        o, l = oa.csa_attend(f64(x["q"][b, 0]), f64(x["entries"][b, rows]), np.arange(rows.size),
                             f64(x["win_rows"][b]), int(x["win_pos0"][b]), tb, w.window, w.rope_dim,
                             1.0 / math.sqrt(w.d))
        ref_o.append(o)
        ref_l.append(l)
    assert_close(out[:, 0], np.stack(ref_o), "out")
    assert_close(lse[:, 0], np.stack(ref_l), "lse")


def test_chain_csa_decode_32k():
    _chain(gen.CSA_DECODE_32K, gen.CSA_DECODE_32K.B)


def test_chain_csa_decode_128k():
    _chain(gen.CSA_DECODE_128K, gen.CSA_DECODE_128K.B)


def test_chain_csa_decode_1m_mxfp4():
    _chain(gen.CSA_DECODE_1M, gen.CSA_DECODE_1M.B)
