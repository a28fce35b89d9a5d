"""Indexer keys produced by compression (csa_compress_index_keys, csa_decode_append_index) against
the oracle: the pooled keys (bf16) within the entry tolerance, and the stored codes equal to the
oracle's quantisation of those same bf16 keys (the quantisation decision taken on one value)."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_03_amd import inputs as gen
from compressed_sparse_attention_03_amd import ops
from oracle import indexer as oi
from oracle import quant as oq
from helpers import assert_close, dev, dev_bf16, f64, host_f64, say

pytestmark = pytest.mark.gpu
CFG = 41


def _stored(keys_f64, fmt):
    """The oracle's storage form of keys, in the library's layout."""
    codes, scales = oi.quantize_keys(keys_f64, fmt)
    if fmt == "fp8":
        return codes.astype(np.uint8), scales.astype(np.float32)
    if fmt == "mxfp4":
        return oq.pack_fp4(codes.astype(np.uint8)), scales.astype(np.uint8)
    return codes.astype(np.float32), None


def _check_codes(kc, ks, keys_gpu, fmt, what):
    codes, scales = _stored(keys_gpu, fmt)
    assert np.array_equal(kc, codes), f"{what}: codes"
    if scales is not None:
        assert np.array_equal(ks, scales), f"{what}: scales"


@pytest.mark.parametrize("B,n_new,D_I,m,overlap,fmt,pos0", [
    (2, 64, 128, 4, 1, "fp8", 0),
    (1, 4096, 128, 4, 1, "mxfp4", 0),          # the prefill chunk's keys
    (2, 256, 128, 4, 1, "f32", 128),           # continuing a sequence: the previous group as halo
    (2, 512, 256, 8, 0, "mxfp4", 0),
    (1, 1024, 128, 128, 0, "fp8", 0),
    (3, 96, 512, 3, 1, "fp8", 6),
    (1, 64, 1024, 4, 0, "mxfp4", 0),
])
def test_compressed_index_keys(B, n_new, D_I, m, overlap, fmt, pos0):
    halo = m if (overlap and pos0 > 0) else 0
    rows = halo + n_new
    say(f"case: compress_index_keys B={B} n_new={n_new} D_I={D_I} m={m} overlap={overlap} fmt={fmt} pos0={pos0}")
    c = gen.normal_bf16(CFG, gen.T_KIDX, (B * rows, D_I)).reshape(B, rows, D_I)
    z = gen.normal_bf16(CFG, gen.T_Z, (B * rows, D_I)).reshape(B, rows, D_I)
    bias = gen.normal_bf16(CFG, gen.T_BIAS, ((1 + overlap) * m, D_I), std=0.1)
    codes, scales, keys = ops.csa_compress_index_keys(dev_bf16(c), dev_bf16(z), dev_bf16(bias), m=m, overlap=overlap,
                                                      key_format=fmt, pos0=pos0, keys_out=True)
    torch.cuda.synchronize()
    kg = host_f64(keys)
    kc = codes.cpu().numpy()
    ks = scales.cpu().numpy() if scales is not None else None
    for b in range(B):
        ref, lo = oi.compress_keys(f64(c[b]), f64(z[b]), f64(bias), m, overlap, pos_first=pos0 - halo)
        assert lo == pos0 // m and ref.shape[0] == n_new // m
        assert_close(kg[b], ref, f"seq {b} keys")
        _check_codes(kc[b], ks[b] if ks is not None else None, kg[b], fmt, f"seq {b}")


@pytest.mark.parametrize("D_I,m,overlap,fmt,steps,offs", [
    (128, 4, 1, "fp8", 40, (0, 5, 11)),
    (128, 4, 1, "mxfp4", 37, (0, 2, 29)),
    (256, 8, 0, "f32", 40, (0, 9, 3)),
])
def test_decode_append_index(D_I, m, overlap, fmt, steps, offs):
    # sequences continue from different positions (their rings and key caches set up from the
    # oracle), take one token per call, and the key cache is compared with the oracle's
    say(f"case: decode_append_index D_I={D_I} m={m} overlap={overlap} fmt={fmt} steps={steps} offs={offs}")
    B, R = len(offs), (1 + overlap) * m
    T = max(offs) + steps
    c = gen.normal_bf16(CFG, gen.T_KIDX, (B * 1000, D_I))
    z = gen.normal_bf16(CFG, gen.T_Z, (B * 1000, D_I))
    bias = gen.normal_bf16(CFG, gen.T_BIAS, (R, D_I), std=0.1)
    seq = [(c[1000 * b:1000 * b + T], z[1000 * b:1000 * b + T]) for b in range(B)]
    N_cap = T // m + 2
    f = ops.KEY_FORMATS[fmt]
    cs, ss = ops._key_cache_shapes((B, N_cap), D_I, f)
    kc = torch.zeros(cs[0], dtype=cs[1], device="cuda")
    ks = torch.zeros(ss[0], dtype=ss[1], device="cuda") if ss is not None else None
    keys = torch.zeros((B, N_cap, D_I), dtype=torch.bfloat16, device="cuda")
    tc = np.zeros((B, R, D_I), dtype=np.uint16)
    tz = np.zeros((B, R, D_I), dtype=np.uint16)
    kc_h, ks_h, keys_h = kc.cpu().numpy(), ks.cpu().numpy() if ks is not None else None, np.zeros((B, N_cap, D_I), np.uint16)
    for b, off in enumerate(offs):
        for p in range(max(0, off - R), off):
            tc[b, p % R], tz[b, p % R] = seq[b][0][p], seq[b][1][p]
        if off >= m:
            ref, _ = oi.compress_keys(f64(seq[b][0][:off]), f64(seq[b][1][:off]), f64(bias), m, overlap)
            n0 = ref.shape[0]
            kb = gen.f32_to_bf16_bits(ref.astype(np.float32))
            keys_h[b, :n0] = kb
            codes, scales = _stored(f64(kb), fmt)
            kc_h[b, :n0] = codes
            if ks_h is not None:
                ks_h[b, :n0] = scales
    kc.copy_(torch.from_numpy(kc_h))
    if ks is not None:
        ks.copy_(torch.from_numpy(ks_h))
    keys.copy_(dev_bf16(keys_h))
    tc_d, tz_d, bias_d = dev_bf16(tc), dev_bf16(tz), dev_bf16(bias)
    for s in range(steps):
        pos = np.array([o + s for o in offs], dtype=np.int64)
        cn = np.stack([seq[b][0][pos[b]] for b in range(B)])
        zn = np.stack([seq[b][1][pos[b]] for b in range(B)])
        ops.csa_decode_append_index(dev_bf16(cn), dev_bf16(zn), dev(pos), bias_d, m=m, overlap=overlap, tok_c=tc_d,
                                    tok_z=tz_d, key_format=fmt, k_codes=kc, k_scales=ks, keys_out=keys)
    torch.cuda.synchronize()
    kg = host_f64(keys)
    kc_g = kc.cpu().numpy()
    ks_g = ks.cpu().numpy() if ks is not None else None
    for b, off in enumerate(offs):
        t_end = off + steps - 1
        ref, _ = oi.compress_keys(f64(seq[b][0][:t_end + 1]), f64(seq[b][1][:t_end + 1]), f64(bias), m, overlap)
        n = ref.shape[0]
        assert_close(kg[b, :n], ref, f"seq {b} keys")
        _check_codes(kc_g[b, :n], ks_g[b, :n] if ks_g is not None else None, kg[b, :n], fmt, f"seq {b}")
        assert (kc_g[b, n:] == 0).all(), f"seq {b}: key rows past the last complete entry were written"
