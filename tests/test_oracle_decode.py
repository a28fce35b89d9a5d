"""Pins of the oracle's decode-cache state against facts outside it: closed-form entry counts,
causality (an entry never changes once written), the window's position range, a constant sequence
(entries coincide with window rows at the entry position), and the stored keys decoding to the
right rows within the formats' error bounds."""
import numpy as np
import pytest

from oracle import decode as od
from oracle import indexer as oi

RNG = np.random.default_rng(11)


def _bf16(x):
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    u = ((u.astype(np.uint64) + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16).astype(np.uint32)
    return u.view(np.float32).astype(np.float64)


def _seq(T, d, m, overlap, d_i=32):
    c = _bf16(RNG.standard_normal((T, d)))
    z = _bf16(RNG.standard_normal((T, d)))
    bias = _bf16(0.1 * RNG.standard_normal(((1 + overlap) * m, d)))
    keys = _bf16(RNG.standard_normal((T // m + 1, d_i)))
    return c, z, bias, keys


@pytest.mark.parametrize("m,overlap,window", [(4, 1, 8), (4, 0, 5), (8, 0, 16), (3, 1, 4)])
def test_counts_window_and_causality(m, overlap, window):
    T, d = 40, 32
    c, z, bias, keys = _seq(T, d, m, overlap)
    prev = None
    for t in range(T):
        st = od.cache_after(c, z, bias, keys, t, m=m, overlap=overlap, rope_dim=8, window=window)
        assert st["n_entries"] == (t + 1) // m                      # closed form
        lo = max(0, t - window + 1)
        assert list(st["win_pos"]) == list(range(lo, t + 1))        # the last `window` positions
        if prev is not None:
            n0 = prev["n_entries"]
            # a new entry appears exactly when position t closes a group
            assert st["n_entries"] - n0 == (1 if (t + 1) % m == 0 else 0)
            # entries already written do not change when later tokens arrive
            assert np.array_equal(st["entries"][:n0], prev["entries"])
            # a window row depends on its own token and position only
            common = np.intersect1d(prev["win_pos"], st["win_pos"])
            a = prev["win_rows"][np.searchsorted(prev["win_pos"], common)]
            b = st["win_rows"][np.searchsorted(st["win_pos"], common)]
            assert np.array_equal(a, b)
        prev = st


@pytest.mark.parametrize("m,overlap", [(4, 1), (8, 0)])
def test_constant_sequence_entries_equal_window_rows(m, overlap):
    # A constant token row compresses to itself (the pooling weights sum to one), and an entry is
    # normalised and rotated at i*m like the window row of that position: the two must coincide.
    T, d = 33, 32
    v = _bf16(RNG.standard_normal(d))
    c = np.tile(v, (T, 1))
    z = _bf16(RNG.standard_normal((T, d)))
    bias = _bf16(0.1 * RNG.standard_normal(((1 + overlap) * m, d)))
    st = od.cache_after(c, z, bias, None, T - 1, m=m, overlap=overlap, rope_dim=8, window=T)
    for i in range(st["n_entries"]):
        row = st["win_rows"][list(st["win_pos"]).index(i * m)]
        np.testing.assert_allclose(st["entries"][i], row, rtol=0, atol=1e-12)


@pytest.mark.parametrize("fmt,rel", [("fp8", 2.0 ** -4), ("mxfp4", None), ("f32", 0.0)])
def test_stored_keys_decode_to_the_entries_keys(fmt, rel):
    m, T = 4, 37
    c, z, bias, keys = _seq(T, 32, m, 1, d_i=64)
    st = od.cache_after(c, z, bias, keys, T - 1, m=m, overlap=1, rope_dim=8, window=8, key_format=fmt)
    n = st["n_entries"]
    dec = oi.dequantize_keys(st["key_codes"], st["key_scales"], fmt)
    assert dec.shape == (n, 64)
    ref = keys[:n]
    if fmt == "mxfp4":
        # e2m1 with a block scale 2^(floor(log2 amax) - 2): a step of at most one quarter of the
        # block's largest magnitude (values up to 6 * 2^s are covered, the grid spacing is <= 2^s)
        for blk in range(2):
            sl = slice(32 * blk, 32 * blk + 32)
            amax = np.abs(ref[:, sl]).max(axis=1, keepdims=True)
            assert np.all(np.abs(dec[:, sl] - ref[:, sl]) <= 0.25 * amax + 1e-12)
    else:
        assert np.all(np.abs(dec - ref) <= rel * np.abs(ref) + 1e-30)
    # a key row shifted by one entry would be far off
    if n > 1:
        assert np.abs(dec[1:] - keys[: n - 1]).max() > 0.5
