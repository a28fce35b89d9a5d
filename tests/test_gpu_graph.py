"""The decode step replayed from a captured HIP graph (as the benchmark times it): every replay,
with eager library calls and poisoned outputs in between, gives the bits of the eager call.  The
library records no memset nodes; the only state its workspaces carry from one call to the next
are the arrival counters, which every completed call leaves at zero (so replays, which share the
eager calls' workspace here, must keep working)."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_03_amd import inputs as gen
from compressed_sparse_attention_03_amd import ops
from helpers import dev, dev_bf16, say

pytestmark = pytest.mark.gpu
REPLAYS = 4


def _csa_step(x, codes, scales, w, sel, out, ws_i, ws_a):
    ops.csa_index_topk(x["q_idx"], x["w_idx"], codes, scales, key_format=w.key_format, n_entries=x["n_entries"],
                       q_pos0=x["t"], m=w.m, topk=w.topk, workspace=ws_i, topk_out=sel)
    ops.csa_attend(x["q"], x["entries"], sel, x["win_rows"], x["win_pos0"], x["t"], rope_dim=w.rope_dim,
                   window=w.window, workspace=ws_a, out=out)


def test_csa_decode_step_graph_replays_match_eager():
    w = gen.CSA_DECODE_32K
    nb = 4
    say(f"case: graph replay csa decode 32k B={nb}")
    h = gen.decode_inputs(w, 0, nb)
    x = {"q_idx": dev_bf16(h["q_idx"]), "w_idx": dev(h["w_idx"]), "n_entries": dev(h["n_entries"]),
         "t": dev(h["t"]), "q": dev_bf16(h["q"]), "entries": dev_bf16(h["entries"]),
         "win_rows": dev_bf16(h["win_rows"]), "win_pos0": dev(h["win_pos0"])}
    codes, scales = ops.csa_quantize_keys(dev_bf16(h["k_idx"]), w.key_format)
    B, Sq, H, D = x["q"].shape
    N = x["entries"].shape[1]
    ws_i = ops.index_topk_workspace(B, Sq, N, w.topk)
    ws_a = ops.attend_workspace(B, Sq, H, D, w.topk, w.window)
    sel = torch.empty((B, Sq, w.topk), dtype=torch.int32, device="cuda")
    out = torch.empty_like(x["q"])
    # eager reference (its own buffers)
    sel_ref = torch.empty_like(sel)
    out_ref = torch.empty_like(out)
    _csa_step(x, codes, scales, w, sel_ref, out_ref, ws_i, ws_a)
    torch.cuda.synchronize()
    # capture on a side stream, then replay with eager work and poisoned outputs in between
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _csa_step(x, codes, scales, w, sel, out, ws_i, ws_a)           # warm-up outside the graph
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            _csa_step(x, codes, scales, w, sel, out, ws_i, ws_a)
    torch.cuda.synchronize()
    scratch_sel, scratch_out = torch.empty_like(sel), torch.empty_like(out)
    for r in range(REPLAYS):
        sel.fill_(-7)
        out.zero_()
        _csa_step(x, codes, scales, w, scratch_sel, scratch_out, ws_i, ws_a)   # eager use of the workspaces
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(sel, sel_ref), f"replay {r}: top-k differs from the eager call"
        assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16)), f"replay {r}: output differs"


def test_hca_decode_step_graph_replays_match_eager():
    w = gen.HCA_DECODE_1M
    nb = 2
    say(f"case: graph replay hca decode B={nb} (4,096 of the entries)")
    h = gen.decode_inputs(w, 0, nb, n_rows=4096, parts=("attend",))
    q, ent, win = dev_bf16(h["q"]), dev_bf16(h["entries"]), dev_bf16(h["win_rows"])
    n_ent = dev(np.full(nb, 4096, np.int64))
    t = dev(np.full(nb, 4096 * w.m + 7, np.int64))
    wp0 = dev(np.full(nb, 4096 * w.m + 8 - w.window, np.int64))
    B, Sq, H, D = q.shape
    ws = ops.hca_workspace(B, Sq, H, D, ent.shape[1], w.window)
    kw = dict(m=w.m, rope_dim=w.rope_dim, window=w.window, workspace=ws)
    ref, _ = ops.hca_attend(q, ent, n_ent, win, wp0, t, **kw)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ops.hca_attend(q, ent, n_ent, win, wp0, t, out=out, **kw)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            ops.hca_attend(q, ent, n_ent, win, wp0, t, out=out, **kw)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        out.zero_()
        ops.hca_attend(q, ent, n_ent, win, wp0, t, **kw)                # eager use of the workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {r}: output differs"
