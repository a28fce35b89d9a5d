"""csa_attend_noalloc (the library's own scratch, no workspace argument) against csa_attend.

Both run the same kernels over the same plan, so their outputs must agree bit for bit.  Two calls
in a row, the second smaller, so the second reads scratch the first left behind only where it
rewrote it itself."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_03_amd import inputs as gen
from compressed_sparse_attention_03_amd import ops
from helpers import dev, dev_bf16, say

pytestmark = pytest.mark.gpu


def _case(cfg, B, H, D, N, k, W):
    g = np.random.default_rng(cfg)
    q = gen.normal_bf16(cfg, 0, (B * H, D)).reshape(B, 1, H, D)
    ent = gen.normal_bf16(cfg, 1, (B * N, D)).reshape(B, N, D)
    win = gen.normal_bf16(cfg, 2, (B * W, D)).reshape(B, W, D)
    sel = np.full((B, 1, k), -1, dtype=np.int32)
    for b in range(B):
        n = min(k - 3, N)
        sel[b, 0, :n] = np.sort(g.choice(N, n, replace=False))
    t = np.full(B, 4 * N - 1, dtype=np.int64)
    return (dev_bf16(q), dev_bf16(ent), dev(sel), dev_bf16(win), dev(t - W + 1), dev(t))


def _both(args, rope, W):
    q = args[0]
    ref_o, ref_l = ops.csa_attend(*args, rope_dim=rope, window=W, lse=True)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    ops.csa_attend_noalloc(*args, rope_dim=rope, window=W, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return ref_o, ref_l, out, lse


def test_noalloc_matches_csa_attend_on_two_calls_the_second_smaller():
    # first: 8 decode queries of 64 x 512 heads over 1,024 + 128 rows, split-K (4.2 MB of partials);
    # second: 2 queries of 16 x 128 heads over 256 + 64 rows, split-K into far less of the scratch
    cases = [(dict(B=8, H=64, D=512, N=20000, k=1024, W=128), 64),
             (dict(B=2, H=16, D=128, N=3000, k=256, W=64), 32)]
    for i, (shape, rope) in enumerate(cases):
        say(f"case: csa_attend_noalloc call {i} {shape}")
        need = ops.lib().csa_attend_workspace_bytes(shape["B"], 1, shape["H"], shape["D"], shape["k"], shape["W"])
        assert need > 256, "the case must run split-K so that the scratch is used"
        ref_o, ref_l, out, lse = _both(_case(90 + i, **shape), rope, shape["W"])
        assert torch.equal(out, ref_o), f"call {i}: output differs from csa_attend"
        assert torch.equal(lse, ref_l), f"call {i}: lse differs from csa_attend"


def test_noalloc_without_split_and_rejection_of_oversized_shapes():
    # 512 queries take the fused plan (no partials at all); then a shape whose partials exceed the
    # scratch is refused before anything is launched
    say("case: csa_attend_noalloc fused plan B=512 H=16 D=128 k=512 W=64")
    ref_o, ref_l, out, lse = _both(_case(93, B=512, H=16, D=128, N=2000, k=512, W=64), 32, 64)
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
    say("case: csa_attend_noalloc oversized B=16 H=128 D=512 k=2048 W=512")
    assert ops.lib().csa_attend_workspace_bytes(16, 1, 128, 512, 2048, 512) > (32 << 20)
    args = _case(94, B=16, H=128, D=512, N=4000, k=2048, W=512)
    out = torch.empty_like(args[0])
    with pytest.raises(RuntimeError, match="scratch"):
        ops.csa_attend_noalloc(*args, rope_dim=64, window=512, out=out)
