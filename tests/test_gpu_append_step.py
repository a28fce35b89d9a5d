"""csa_decode_append_step (both streams of a decode step's cache maintenance in one launch) against
csa_decode_append (KV stream, no k_new) followed by csa_decode_append_index (indexer stream).

The fused launch runs the same per-sequence code as the two calls, so every cache must come out
bit-identical after every step: entries, window ring, both token rings, the indexer keys (bf16 copy,
codes and scales) and n_entries.  The oracle comparison of that code is test_gpu_append.py's and
test_gpu_index_keys.py's."""
import pytest
import torch

from compressed_sparse_attention_03_amd import ops
from helpers import say

pytestmark = pytest.mark.gpu


def _caches(B, d, D_I, m, overlap, W_cap, N_cap, fmt, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    bf = lambda *s, std=1.0: (std * torch.randn(s, generator=g, device="cuda")).to(torch.bfloat16)
    R = (1 + overlap) * m
    c = {"tok_c": bf(B, R, d), "tok_z": bf(B, R, d), "win_ring": bf(B, W_cap, d), "entries": bf(B, N_cap, d),
         "n_entries": torch.zeros(B, dtype=torch.int64, device="cuda"), "tok_ci": bf(B, R, D_I),
         "tok_zi": bf(B, R, D_I), "keys_out": bf(B, N_cap, D_I)}
    if fmt == "fp8":
        c["k_codes"] = torch.zeros((B, N_cap, D_I), dtype=torch.uint8, device="cuda")
        c["k_scales"] = torch.zeros((B, N_cap), dtype=torch.float32, device="cuda")
    elif fmt == "mxfp4":
        c["k_codes"] = torch.zeros((B, N_cap, D_I // 2), dtype=torch.uint8, device="cuda")
        c["k_scales"] = torch.zeros((B, N_cap, D_I // 32), dtype=torch.uint8, device="cuda")
    else:
        c["k_codes"] = torch.zeros((B, N_cap, D_I), dtype=torch.float32, device="cuda")
        c["k_scales"] = None
    return c, bf


@pytest.mark.parametrize("d,D_I,m,overlap,fmt,W_cap,N_cap,steps,starts", [
    (512, 128, 4, 1, "mxfp4", 128, 64, 13, (0, 5, 30, -1)),     # the 1M decode shapes, one idle sequence
    (128, 128, 4, 1, "fp8", 16, 40, 10, (2, 3, 7)),
    (256, 256, 8, 0, "f32", 8, 16, 20, (0, 11)),
    (1024, 512, 3, 1, "mxfp4", 5, 20, 9, (0, 1)),
    (512, 128, 128, 0, "fp8", 128, 4, 260, (0, 129)),           # HCA-like groups: 128 tokens
])
def test_fused_step_equals_the_two_calls(d, D_I, m, overlap, fmt, W_cap, N_cap, steps, starts):
    say(f"case: decode_append_step d={d} D_I={D_I} m={m} overlap={overlap} fmt={fmt} steps={steps} starts={starts}")
    B = len(starts)
    fused, bf = _caches(B, d, D_I, m, overlap, W_cap, N_cap, fmt, 7)
    split = {k: (v.clone() if v is not None else None) for k, v in fused.items()}
    R = (1 + overlap) * m
    bias, bias_i, norm_w = bf(R, d, std=0.1), bf(R, D_I, std=0.1), bf(d, std=0.2) + 1.0
    for s in range(steps):
        pos = torch.tensor([p + s if p >= 0 else -1 for p in starts], dtype=torch.int64, device="cuda")
        c_new, z_new, ci_new, zi_new = bf(B, d), bf(B, d), bf(B, D_I), bf(B, D_I)
        ops.csa_decode_append_step(c_new, z_new, pos, bias, m=m, overlap=overlap, rope_dim=64, norm_w=norm_w,
                                   tok_c=fused["tok_c"], tok_z=fused["tok_z"], win_ring=fused["win_ring"],
                                   entries=fused["entries"], n_entries=fused["n_entries"], c_i_new=ci_new,
                                   z_i_new=zi_new, bias_i=bias_i, tok_ci=fused["tok_ci"], tok_zi=fused["tok_zi"],
                                   key_format=fmt, k_codes=fused["k_codes"], k_scales=fused["k_scales"],
                                   keys_out=fused["keys_out"])
        ops.csa_decode_append(c_new, z_new, pos, bias, m=m, overlap=overlap, rope_dim=64, norm_w=norm_w,
                              tok_c=split["tok_c"], tok_z=split["tok_z"], win_ring=split["win_ring"],
                              entries=split["entries"], n_entries=split["n_entries"])
        ops.csa_decode_append_index(ci_new, zi_new, pos, bias_i, m=m, overlap=overlap, tok_c=split["tok_ci"],
                                    tok_z=split["tok_zi"], key_format=fmt, k_codes=split["k_codes"],
                                    k_scales=split["k_scales"], keys_out=split["keys_out"])
        torch.cuda.synchronize()
        for k, v in fused.items():
            if v is not None:
                assert torch.equal(v, split[k]), f"step {s}: {k} differs"
    # n_entries: the last entry closed inside the run (entries at N_cap or beyond are dropped)
    want = []
    for p in starts:
        closed = [(t + 1) // m for t in range(p, p + steps) if p >= 0 and (t + 1) % m == 0 and (t + 1) // m <= N_cap]
        want.append(closed[-1] if closed else 0)
    assert fused["n_entries"].cpu().tolist() == want
