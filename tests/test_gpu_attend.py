"""GPU core attention (csa_attend / hca_attend) vs the oracle."""
import math

import numpy as np
import pytest
import torch

from compressed_sparse_attention_03_amd import inputs as gen
from compressed_sparse_attention_03_amd import ops
from oracle import attention as oa
from helpers import assert_close, dev, dev_bf16, f64, host_f64, say

pytestmark = pytest.mark.gpu


def _selection(g, B, Sq, N, k, n_pad=0):
    sel = np.full((B, Sq, k), -1, dtype=np.int32)
    for b in range(B):
        for s in range(Sq):
            n = min(k - n_pad, N)
            sel[b, s, :n] = np.sort(g.choice(N, n, replace=False))
    return sel


def check_csa(q, entries, sel, win_rows, win_pos0, t_first, window, rope_dim, tag, q_norm_w=None,
              sample=None):
    """q [B,Sq,H,D] u16, entries [B,N,D] u16, sel [B,Sq,k] int32, win_rows [B,W,D] u16."""
    B, Sq, H, D = q.shape
    say(f"case: csa_attend {tag} B={B} Sq={Sq} H={H} D={D} k={sel.shape[2]} W={window}")
    nw = dev_bf16(q_norm_w) if q_norm_w is not None else None
    out, lse = ops.csa_attend(dev_bf16(q), dev_bf16(entries), dev(sel), dev_bf16(win_rows),
                              dev(np.asarray(win_pos0, np.int64)), dev(np.asarray(t_first, np.int64)),
                              rope_dim=rope_dim, window=window, q_norm_w=nw, lse=True)
    out, lse = host_f64(out), host_f64(lse)
    gw = f64(q_norm_w) if q_norm_w is not None else None
    ref_o, got_o, ref_l, got_l = [], [], [], []
    for b in range(B):
        win_b = f64(win_rows[b])
        for s in (range(Sq) if sample is None else sample):
            rows = sel[b, s][sel[b, s] >= 0]
            sub = f64(entries[b, rows]) if rows.size else np.zeros((1, D))
            o, l = oa.csa_attend(f64(q[b, s]), sub, np.arange(rows.size), win_b, int(win_pos0[b]),
                                 int(t_first[b] + s), window, rope_dim, 1.0 / math.sqrt(D), gw)
            ref_o.append(o); got_o.append(out[b, s]); ref_l.append(l); got_l.append(lse[b, s])
    assert_close(np.stack(got_o), np.stack(ref_o), "out")
    assert_close(np.stack(got_l), np.stack(ref_l), "lse")


def _rand_case(cfg, B, Sq, H, D, N, k, W, n_pad=0, t_first=None, win_pos0=None, Wcap=None):
    g = np.random.default_rng(cfg)
    q = gen.normal_bf16(cfg, 0, (B * Sq * H, D)).reshape(B, Sq, H, D)
    ent = gen.normal_bf16(cfg, 1, (B * N, D)).reshape(B, N, D)
    Wcap = W if Wcap is None else Wcap
    win = gen.normal_bf16(cfg, 2, (B * Wcap, D)).reshape(B, Wcap, D)
    sel = _selection(g, B, Sq, N, k, n_pad)
    t_first = np.full(B, 4 * N - 1) if t_first is None else np.asarray(t_first)
    win_pos0 = t_first - W + 1 if win_pos0 is None else np.asarray(win_pos0)
    return q, ent, sel, win, win_pos0, t_first


@pytest.mark.parametrize("H,D,rope", [(64, 512, 64), (8, 64, 16), (24, 128, 32), (16, 256, 0)])
def test_shapes(H, D, rope):
    q, ent, sel, win, wp, tf = _rand_case(70, 3, 1, H, D, 3000, 256, 64, n_pad=5)
    check_csa(q, ent, sel, win, wp, tf, 64, rope, f"H{H}D{D}")


def test_window_clipped_at_sequence_start_and_empty_selection():
    # queries at t = 0..5 see 1..6 window rows; the first ones select nothing
    B, Sq, H, D, W = 1, 6, 16, 128, 32
    q, ent, sel, win, wp, tf = _rand_case(71, B, Sq, H, D, 64, 8, W, t_first=[0], win_pos0=[0], Wcap=64)
    sel[0, :3] = -1
    check_csa(q, ent, sel, win, wp, tf, W, 32, "early")


def test_norm_weight_and_split_with_only_padding():
    # k = 2048 with 1900 empty slots: some row slices hold no row at all
    q, ent, sel, win, wp, tf = _rand_case(72, 2, 1, 64, 512, 5000, 2048, 128, n_pad=1900)
    nw = gen.normal_bf16(72, 5, (1, 512), std=0.2, mean=1.0)[0]
    check_csa(q, ent, sel, win, wp, tf, 128, 64, "pad", q_norm_w=nw)


def test_csa_decode_32k_full():
    w = gen.CSA_DECODE_32K
    x = gen.decode_inputs(w, parts=("attend",))
    sel = _selection(np.random.default_rng(73), w.B, 1, w.N, w.topk)
    check_csa(x["q"], x["entries"], sel, x["win_rows"], x["win_pos0"], x["t"], w.window, w.rope_dim, w.name)


def test_csa_decode_1m_full():
    w = gen.CSA_DECODE_1M
    x = gen.decode_inputs(w, parts=("attend",))
    sel = _selection(np.random.default_rng(74), w.B, 1, w.N, w.topk)
    check_csa(x["q"], x["entries"], sel, x["win_rows"], x["win_pos0"], x["t"], w.window, w.rope_dim, w.name)


def test_csa_decode_1m_flash_topk512_full():
    w = gen.CSA_DECODE_1M_FLASH
    x = gen.decode_inputs(w, parts=("attend",))
    sel = _selection(np.random.default_rng(75), w.B, 1, w.N, w.topk)
    check_csa(x["q"], x["entries"], sel, x["win_rows"], x["win_pos0"], x["t"], w.window, w.rope_dim, w.name)


def test_hca_decode_1m_full():
    w = gen.HCA_DECODE_1M
    x = gen.decode_inputs(w, parts=("attend",))
    say(f"case: hca_attend {w.name}")
    out, lse = ops.hca_attend(dev_bf16(x["q"]), dev_bf16(x["entries"]), dev(x["n_entries"]),
                              dev_bf16(x["win_rows"]), dev(x["win_pos0"]), dev(x["t"]), m=w.m,
                              rope_dim=w.rope_dim, window=w.window, lse=True)
    out, lse = host_f64(out), host_f64(lse)
    ro, rl = [], []
    for b in range(w.B):
        o, l = oa.hca_attend(f64(x["q"][b, 0]), f64(x["entries"][b]), w.N, f64(x["win_rows"][b]),
                             int(x["win_pos0"][b]), int(x["t"][b]), w.window, w.rope_dim)
        ro.append(o); rl.append(l)
    assert_close(out[:, 0], np.stack(ro), "hca out")
    assert_close(lse[:, 0], np.stack(rl), "hca lse")


def test_hca_causal_prefix_and_equals_csa_with_all_entries():
    B, Sq, H, D, N, W = 2, 3, 16, 256, 300, 16
    cfg = 75
    q = gen.normal_bf16(cfg, 0, (B * Sq * H, D)).reshape(B, Sq, H, D)
    ent = gen.normal_bf16(cfg, 1, (B * N, D)).reshape(B, N, D)
    win = gen.normal_bf16(cfg, 2, (B * 64, D)).reshape(B, 64, D)
    m = 8
    tf = np.array([8 * 100 - 2, 8 * 400], dtype=np.int64)      # sequence 0 sees 99..100 entries
    wp = tf - 40
    n_ent = np.array([N, 250], dtype=np.int64)
    say("case: hca causal prefix")
    out, _ = ops.hca_attend(dev_bf16(q), dev_bf16(ent), dev(n_ent), dev_bf16(win), dev(wp), dev(tf), m=m,
                            rope_dim=32, window=W)
    # the same through csa_attend with the visible prefix as the selection
    sel = np.full((B, Sq, N), -1, dtype=np.int32)
    for b in range(B):
        for s in range(Sq):
            nv = min(n_ent[b], (tf[b] + s + 1) // m)
            sel[b, s, :nv] = np.arange(nv)
    out2, _ = ops.csa_attend(dev_bf16(q), dev_bf16(ent), dev(sel), dev_bf16(win), dev(wp), dev(tf),
                             rope_dim=32, window=W)
    assert_close(host_f64(out), host_f64(out2), "hca vs csa(all)", max_abs=1e-2, mean_abs=1e-3)
    check_csa(q, ent, sel, win, wp, tf, W, 32, "hca-as-csa")


def test_prefill_attention_full_size_sampled():
    # 4,096 causal queries at positions 131,072.. with their own selections over the visible
    # entries; the window rows hold 127 earlier tokens plus the chunk.
    w = gen.CSA_PREFILL_128K
    Sq, H, D, W, k = w.Sq, w.H, w.d, w.window, w.topk
    N = w.N + Sq // w.m
    cfg = 76
    q = gen.normal_bf16(cfg, 0, (Sq * H, D)).reshape(1, Sq, H, D)
    ent = gen.normal_bf16(cfg, 1, (N, D)).reshape(1, N, D)
    win = gen.normal_bf16(cfg, 2, (Sq + W - 1, D)).reshape(1, Sq + W - 1, D)
    g = np.random.default_rng(cfg)
    sel = np.empty((1, Sq, k), dtype=np.int32)
    for s in range(Sq):
        nv = (w.T + s + 1) // w.m
        sel[0, s] = np.sort(g.choice(nv, k, replace=False))
    tf = np.array([w.T])
    wp = np.array([w.T - W + 1])
    sample = sorted(set([0, 1, 2, 3, Sq - 1] + g.integers(0, Sq, 40).tolist()))
    check_csa(q, ent, sel, win, wp, tf, W, w.rope_dim, "prefill", sample=sample)


def test_deterministic_repeat():
    q, ent, sel, win, wp, tf = _rand_case(77, 4, 1, 64, 512, 4000, 1024, 128)
    args = (dev_bf16(q), dev_bf16(ent), dev(sel), dev_bf16(win), dev(wp), dev(tf))
    a, la = ops.csa_attend(*args, rope_dim=64, window=128, lse=True)
    b, lb = ops.csa_attend(*args, rope_dim=64, window=128, lse=True)
    assert torch.equal(a, b) and torch.equal(la, lb)


@pytest.mark.parametrize("D", [64, 128])
def test_hca_long_list_many_slices(D):
    """A list of 70,032 rows is cut into 35 slices of 2,048: more than one window of slice
    log2-sum-exps in the combine (16 at D = 64, 32 at D = 128); against the oracle."""
    B, Sq, H, N, W, m = 1, 1, 8, 70000, 32, 4
    cfg = 76
    q = gen.normal_bf16(cfg, 0, (B * Sq * H, D)).reshape(B, Sq, H, D)
    ent = gen.normal_bf16(cfg, 1, (B * N, D)).reshape(B, N, D)
    win = gen.normal_bf16(cfg, 2, (B * W, D)).reshape(B, W, D)
    t = np.array([m * N + 3], dtype=np.int64)                    # every entry visible
    wp = t - W + 1
    n_ent = np.array([N], dtype=np.int64)
    say(f"case: hca long list D={D} N={N} (35 slices)")
    out, lse = ops.hca_attend(dev_bf16(q), dev_bf16(ent), dev(n_ent), dev_bf16(win), dev(wp), dev(t), m=m,
                              rope_dim=16, window=W, lse=True)
    ref_o, ref_l = oa.hca_attend(f64(q[0, 0]), f64(ent[0]), N, f64(win[0]), int(wp[0]), int(t[0]), W, 16,
                                 1.0 / math.sqrt(D))
    assert_close(host_f64(out)[0, 0], ref_o, "out")
    assert_close(host_f64(lse)[0, 0], ref_l, "lse")
