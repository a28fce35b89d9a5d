"""Oracle step 2a: low-precision encodings used by the lightning indexer.

[DEVTO] "Two Compression Strategies": the lightning indexer runs in FP4 precision.
[RABBIT] lightning-indexer paragraph: compact, low-precision operands are what keep the
indexer's first pass cheap.

Two encodings are provided: fp8 e4m3 (OCP "E4M3FN": bias 7, no infinities, 448 largest finite)
with one power-of-two scale per row, and MXFP4 (OCP Microscaling v1.0: e2m1 elements with one
e8m0 power-of-two scale per block of 32).  The element codecs are written from the format
definitions; rounding picks the nearest representable magnitude (ties to the even code) and
saturates at the largest finite magnitude, keeping the sign bit of the input.
Test infrastructure only.
"""
from __future__ import annotations

import numpy as np

FP8_MAX = 448.0
FP4_MAX = 6.0
MX_BLOCK = 32


def fp8_e4m3_value(code: int) -> float:
    """Value of one e4m3 code: sign | 4-bit exponent (bias 7) | 3-bit mantissa; S.1111.111 = NaN."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    f = code & 0x7
    if e == 0xF and f == 0x7:
        return float("nan")
    if e == 0:
        return s * (f / 8.0) * 2.0 ** -6
    return s * (1.0 + f / 8.0) * 2.0 ** (e - 7)


FP8_TABLE = np.array([fp8_e4m3_value(c) for c in range(256)])


def fp4_e2m1_value(code: int) -> float:
    """Value of one e2m1 code: sign | 2-bit exponent (bias 1) | 1-bit mantissa."""
    s = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    f = code & 0x1
    if e == 0:
        return s * f * 0.5
    return s * (1.0 + f / 2.0) * 2.0 ** (e - 1)


FP4_TABLE = np.array([fp4_e2m1_value(c) for c in range(16)])


def _nearest_code(x: np.ndarray, table: np.ndarray, max_code_mag: int) -> np.ndarray:
    """Nearest representable magnitude, ties to the code with an even mantissa LSB, saturating.

    ``table[0..max_code_mag]`` are the non-negative magnitudes in increasing order; the sign is
    applied by the caller.  Values past the largest magnitude saturate to it.
    """
    mags = table[:max_code_mag + 1]
    ax = np.abs(np.asarray(x, dtype=np.float64))
    hi = np.clip(np.searchsorted(mags, ax, side="left"), 0, max_code_mag)
    lo = np.clip(hi - 1, 0, max_code_mag)
    d_lo = np.abs(ax - mags[lo])
    d_hi = np.abs(mags[hi] - ax)
    code = np.where(d_lo < d_hi, lo, hi)
    tie = (d_lo == d_hi) & (lo != hi)
    code = np.where(tie, np.where(lo % 2 == 0, lo, hi), code)
    return code.astype(np.int64)


def fp8_e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round to e4m3 with ties to even, saturating at +-448 (never produces NaN)."""
    x = np.asarray(x, dtype=np.float64)
    mag = _nearest_code(x, FP8_TABLE, 0x7E)
    sign = np.where(np.signbit(x), 0x80, 0)
    return (mag | sign).astype(np.uint8)            # the sign is kept for zero magnitudes too


def fp4_e2m1_encode(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    mag = _nearest_code(x, FP4_TABLE, 0x7)
    sign = np.where(np.signbit(x), 0x8, 0)
    return (mag | sign).astype(np.uint8)


def fp8_row_scale_exp(amax):
    """Smallest e with amax <= 448 * 2**e (clamped to [-126, 127]); 0 for an all-zero row.

    Reading: one power-of-two scale per row, so scaling is exact and the stored scale is 4 bytes.
    Works elementwise on an array of row maxima.
    """
    amax = np.asarray(amax, dtype=np.float64)
    e = np.frexp(amax)[1].astype(np.int64) - 12
    for _ in range(16):
        e = e + (amax / np.exp2(e.astype(np.float64)) > FP8_MAX)
    e = np.clip(e, -126, 127)
    return np.where(amax == 0.0, 0, e)


def quantize_fp8_rows(x: np.ndarray):
    """Per-row fp8: returns (codes uint8 [..., D], scale float64 [...] = 2**e)."""
    x = np.asarray(x, dtype=np.float64)
    e = fp8_row_scale_exp(np.abs(x).max(axis=-1))
    scales = np.exp2(e.astype(np.float64))
    codes = fp8_e4m3_encode(x / scales[..., None])
    return codes, scales


def dequantize_fp8_rows(codes, scales):
    return FP8_TABLE[np.asarray(codes, dtype=np.int64)] * np.asarray(scales, dtype=np.float64)[..., None]


def mx_scale_byte(amax):
    """OCP MX v1.0 shared scale for e2m1: X = 2**(floor(log2 amax) - 2), stored as e8m0.

    The e8m0 byte is the biased exponent (bias 127), clamped to [0, 254]; an all-zero block
    stores 0.  Works elementwise on an array of block maxima.
    """
    amax = np.asarray(amax, dtype=np.float64)
    fl = np.frexp(amax)[1].astype(np.int64) - 1          # floor(log2(amax)) for amax > 0
    b = np.clip(fl - 2 + 127, 0, 254)
    return np.where(amax == 0.0, 0, b).astype(np.uint8)


def quantize_mxfp4(x: np.ndarray):
    """MXFP4 along the last axis (length a multiple of 32).

    Returns (codes uint8 [..., D] one e2m1 code per element, scale bytes uint8 [..., D/32]).
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    assert D % MX_BLOCK == 0
    blocks = x.reshape(x.shape[:-1] + (D // MX_BLOCK, MX_BLOCK))
    sb = mx_scale_byte(np.abs(blocks).max(axis=-1))
    X = np.exp2(sb.astype(np.float64) - 127.0)
    codes = fp4_e2m1_encode(blocks / X[..., None])
    return codes.reshape(x.shape), sb


def dequantize_mxfp4(codes, scale_bytes):
    codes = np.asarray(codes, dtype=np.int64)
    D = codes.shape[-1]
    vals = FP4_TABLE[codes].reshape(codes.shape[:-1] + (D // MX_BLOCK, MX_BLOCK))
    sc = 2.0 ** (np.asarray(scale_bytes, dtype=np.float64) - 127.0)
    return (vals * sc[..., None]).reshape(codes.shape)


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """Two e2m1 codes per byte along the last axis: element 2j in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out
