"""Batch invariance and determinism: a query's attention output has the same bits whether it is
computed alone, inside a batch of decode queries (split-K slices merged by the combine kernel), or
inside a prefill-sized call (one workgroup per query and head block merging the same slices in
the same order); its top-k selection is the same set in any batch; repeated calls are equal."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_03_amd import inputs as gen
from compressed_sparse_attention_03_amd import ops
from oracle import attention as oa
from helpers import assert_close, dev, dev_bf16, f64, host_f64, say

pytestmark = pytest.mark.gpu
CFG = 42
H, D, R, W, K = 64, 512, 64, 128, 1024
N, T0, SQ = 4096, 16384, 600          # entries; position of query 0; queries in the prefill-sized call


def _inputs():
    rng = np.random.default_rng(9)
    ent = gen.normal_bf16(CFG, gen.T_ENTRIES, (N, D))
    win = gen.normal_bf16(CFG, gen.T_WIN, (W + SQ, D))           # window rows of positions T0-W+1 ..
    q = gen.normal_bf16(CFG, gen.T_Q, (SQ * H, D)).reshape(SQ, H, D)
    sel = np.full((SQ, K), -1, dtype=np.int32)
    for s in range(SQ):
        n = K - (s % 7) * 50                                     # some selections padded with -1
        sel[s, :n] = np.sort(rng.choice(N, n, replace=False))
    return ent, win, q, sel


def _csa(ent, win, q, sel, t):
    """One call over B sequences of Sq queries each: ent/win [B, ...], q [B, Sq, H, D], sel [B, Sq, K]."""
    B = q.shape[0]
    out, lse = ops.csa_attend(dev_bf16(q), dev_bf16(ent), dev(sel), dev_bf16(win),
                              dev(np.full(B, T0 - W + 1, np.int64)), dev(np.asarray(t, np.int64)),
                              rope_dim=R, window=W, lse=True)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy(), lse.cpu().numpy()


def test_csa_output_bits_do_not_depend_on_the_batch():
    ent, win, q, sel = _inputs()
    say(f"case: batch invariance csa H={H} D={D} k={K} W={W} prefill Sq={SQ}")
    # a prefill-sized call: one sequence, SQ consecutive queries (fused path)
    o_pre, l_pre = _csa(ent[None], win[None], q[None], sel[None], [T0])
    # decode calls: sixteen sequences (copies of the cache), one query each, at various positions
    picks = [0, 1, 7, 50, 99, 128, 255, 300, 333, 401, 402, 450, 499, 512, 577, SQ - 1]
    B = len(picks)
    o_dec, l_dec = _csa(np.stack([ent] * B), np.stack([win] * B), q[picks][:, None], sel[picks][:, None],
                        [T0 + s for s in picks])
    for i, s in enumerate(picks):
        assert np.array_equal(o_dec[i, 0], o_pre[0, s]), f"query {s}: decode batch vs prefill call"
        assert np.array_equal(l_dec[i, 0], l_pre[0, s]), f"query {s}: lse"
    # one query alone
    for s in (3, 401):
        o1, l1 = _csa(ent[None], win[None], q[s][None, None], sel[s][None, None], [T0 + s])
        assert np.array_equal(o1[0, 0], o_pre[0, s]) and np.array_equal(l1[0, 0], l_pre[0, s]), f"query {s} alone"
    # repeat
    o_rep, l_rep = _csa(ent[None], win[None], q[None], sel[None], [T0])
    assert np.array_equal(o_rep, o_pre) and np.array_equal(l_rep, l_pre), "repeated call differs"
    # and the fused path is right (against the oracle, a sample of queries)
    win_f = f64(win)
    got, ref = [], []
    for s in (0, 123, 599):
        ro, _ = oa.csa_attend(f64(q[s]), f64(ent), sel[s], win_f, T0 - W + 1, T0 + s, W, R, 1.0 / np.sqrt(D))
        got.append(host_f64(torch.from_numpy(o_pre[0, s]).view(torch.bfloat16)))
        ref.append(ro)
    assert_close(np.stack(got), np.stack(ref), "fused path out")


def test_hca_output_bits_do_not_depend_on_the_batch():
    say("case: batch invariance hca")
    ent, win, q, _ = _inputs()
    m = 4
    n_ent = np.array([N], np.int64)

    def call(B, qq, t):
        out, lse = ops.hca_attend(dev_bf16(qq), dev_bf16(np.stack([ent] * B)), dev(np.repeat(n_ent, B)),
                                  dev_bf16(np.stack([win] * B)), dev(np.full(B, T0 - W + 1, np.int64)),
                                  dev(np.asarray(t, np.int64)), m=m, rope_dim=R, window=W, lse=True)
        torch.cuda.synchronize()
        return out.view(torch.int16).cpu().numpy(), lse.cpu().numpy()
    o_pre, l_pre = call(1, q[None], [T0])
    picks = [0, 99, 333, SQ - 1]
    o_dec, l_dec = call(len(picks), q[picks][:, None], [T0 + s for s in picks])
    for i, s in enumerate(picks):
        assert np.array_equal(o_dec[i, 0], o_pre[0, s]) and np.array_equal(l_dec[i, 0], l_pre[0, s]), f"query {s}"


def test_index_selection_does_not_depend_on_the_batch():
    # the selection is exact, so a query's set is the same whatever shares its call (different
    # tile plans for 1 and 16 queries)
    w = gen.CSA_DECODE_32K
    x = gen.decode_inputs(w, parts=("index",))
    say("case: batch invariance index 32k")
    codes, scales = ops.csa_quantize_keys(dev_bf16(x["k_idx"]), w.key_format)
    kw = dict(key_format=w.key_format, m=w.m, topk=w.topk)
    sel_all, _ = ops.csa_index_topk(dev_bf16(x["q_idx"]), dev(x["w_idx"]), codes, scales,
                                    n_entries=dev(x["n_entries"]), q_pos0=dev(x["t"]), **kw)
    sel_all = sel_all.cpu().numpy()
    for b in (0, 5, 15):
        s1, _ = ops.csa_index_topk(dev_bf16(x["q_idx"][b:b + 1]), dev(x["w_idx"][b:b + 1]), codes[b:b + 1].contiguous(),
                                   scales[b:b + 1].contiguous(), n_entries=dev(x["n_entries"][b:b + 1]),
                                   q_pos0=dev(x["t"][b:b + 1]), **kw)
        assert np.array_equal(s1.cpu().numpy()[0], sel_all[b]), f"sequence {b}"


@pytest.mark.parametrize("heads,norm_w", [(48, False), (80, True), (128, False)])
def test_long_list_kernel_bits_equal_the_fused_path(heads, norm_w):
    """A long row list (2,048 selected entries + a 128-row window) at D = 512 is taken by the
    head-shared split kernel for a few queries and by the channel-split fused kernel for many: the
    outputs are bitwise equal, with head counts that leave part of a 64-head group empty or fill two, ragged
    selections and a norm weight; a sample of queries also against the oracle."""
    k_long, sq = 2048, 300
    say(f"case: long-list kernel vs fused path H={heads} D={D} k={k_long} W={W} norm_w={norm_w}")
    rng = np.random.default_rng(17)
    ent = gen.normal_bf16(CFG, gen.T_ENTRIES, (N, D))
    win = gen.normal_bf16(CFG, gen.T_WIN, (W + sq, D))
    q = gen.normal_bf16(CFG, gen.T_Q, (sq * heads, D)).reshape(sq, heads, D)
    wn = gen.normal_bf16(CFG, 5, (1, D), std=0.25, mean=1.0)[0] if norm_w else None     # bf16 bits
    sel = np.full((sq, k_long), -1, dtype=np.int32)
    for s in range(sq):
        n = k_long - (s % 5) * 300
        sel[s, :n] = np.sort(rng.choice(N, n, replace=False))

    def call(B, qq, ss, t):
        out, lse = ops.csa_attend(dev_bf16(qq), dev_bf16(np.stack([ent] * B)), dev(ss), dev_bf16(np.stack([win] * B)),
                                  dev(np.full(B, T0 - W + 1, np.int64)), dev(np.asarray(t, np.int64)),
                                  rope_dim=R, window=W, lse=True, q_norm_w=None if wn is None else dev_bf16(wn))
        torch.cuda.synchronize()
        return out.view(torch.int16).cpu().numpy(), lse.cpu().numpy()
    o_pre, l_pre = call(1, q[None], sel[None], [T0])                     # fused path
    picks = [0, 1, 2, 3, 4, 150, sq - 1]
    o_dec, l_dec = call(len(picks), q[picks][:, None], sel[picks][:, None], [T0 + s for s in picks])
    for i, s in enumerate(picks):
        assert np.array_equal(o_dec[i, 0], o_pre[0, s]), f"query {s}: head-shared split vs fused"
        assert np.array_equal(l_dec[i, 0], l_pre[0, s]), f"query {s}: lse"
    win_f = f64(win)
    got, ref = [], []
    wn_ref = None if wn is None else f64(wn)
    for i, s in enumerate((0, 4)):
        ro, _ = oa.csa_attend(f64(q[s]), f64(ent), sel[s], win_f, T0 - W + 1, T0 + s, W, R, 1.0 / np.sqrt(D),
                              q_norm_w=wn_ref)
        got.append(host_f64(torch.from_numpy(o_dec[picks.index(s), 0]).view(torch.bfloat16)))
        ref.append(ro)
    assert_close(np.stack(got), np.stack(ref), "head-shared kernel out")


def test_long_list_kernel_with_a_window_ring():
    """HCA over 4,096 entries with the window held in a ring (no window start): the head-shared
    split kernel (a few queries) equals the fused path (many queries) bit for bit."""
    sq, ring = 256, 512
    say(f"case: long-list kernel, window ring of {ring} rows, HCA Sq={sq}")
    ent = gen.normal_bf16(CFG, gen.T_ENTRIES, (N, D))
    q = gen.normal_bf16(CFG, gen.T_Q, (sq * H, D)).reshape(sq, H, D)
    rows = gen.normal_bf16(CFG, gen.T_WIN, (ring, D))             # row j holds every position p = j mod ring
    m = 4
    n_ent = np.array([N], np.int64)

    def call(B, qq, t):
        out, lse = ops.hca_attend(dev_bf16(qq), dev_bf16(np.stack([ent] * B)), dev(np.repeat(n_ent, B)),
                                  dev_bf16(np.stack([rows] * B)), None, dev(np.asarray(t, np.int64)),
                                  m=m, rope_dim=R, window=W, lse=True)
        torch.cuda.synchronize()
        return out.view(torch.int16).cpu().numpy(), lse.cpu().numpy()
    o_pre, l_pre = call(1, q[None], [T0])
    picks = [0, 77, sq - 1]
    o_dec, l_dec = call(len(picks), q[picks][:, None], [T0 + s for s in picks])
    for i, s in enumerate(picks):
        assert np.array_equal(o_dec[i, 0], o_pre[0, s]) and np.array_equal(l_dec[i, 0], l_pre[0, s]), f"query {s}"
