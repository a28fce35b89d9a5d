"""Seeded synthetic inputs shared by the HIP path's tests, the benchmark and the oracle's tests.

This module holds no arithmetic of the method itself: it draws random numbers, rounds them to
bf16 storage, and describes the workload shapes.  Everything that the method computes lives
either in the HIP library (product) or in ``oracle/`` (test infrastructure).

Seeding: every tensor is drawn from ``PCG64(SeedSequence([1000 + cfg, tensor_id, chunk]))``
with rows generated in chunks of ``CHUNK_ROWS`` so that a slice of a very long tensor (a 1M-token
sequence) can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK_ROWS = 4096

# Fixed tensor ids (part of the seed): keep this order stable.
T_C, T_Z, T_BIAS, T_Q, T_QIDX, T_W, T_KIDX, T_ENTRIES, T_WIN, T_PLANT = range(10)


def _rng(cfg: int, tensor_id: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000 + cfg, tensor_id, chunk])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 storage (round to nearest even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _draw_rows(cfg, tensor_id, row0, nrows, cols, dist, a, b):
    """Rows [row0, row0+nrows) of a [rows, cols] tensor, drawn chunk by chunk."""
    out = np.empty((nrows, cols), dtype=np.float32)
    c0 = row0 // CHUNK_ROWS
    c1 = (row0 + nrows - 1) // CHUNK_ROWS if nrows > 0 else c0 - 1

    def one(ci):
        g = _rng(cfg, tensor_id, ci)
        if dist == "normal":
            blk = g.standard_normal((CHUNK_ROWS, cols), dtype=np.float32) * np.float32(b) + np.float32(a)
        else:
            blk = g.random((CHUNK_ROWS, cols), dtype=np.float32) * np.float32(b - a) + np.float32(a)
        lo = max(row0, ci * CHUNK_ROWS)
        hi = min(row0 + nrows, (ci + 1) * CHUNK_ROWS)
        out[lo - row0:hi - row0] = blk[lo - ci * CHUNK_ROWS:hi - ci * CHUNK_ROWS]

    chunks = list(range(c0, c1 + 1))
    if len(chunks) > 8:
        with ThreadPoolExecutor(max_workers=8) as ex:
            list(ex.map(one, chunks))
    else:
        for ci in chunks:
            one(ci)
    return out


def normal_f32(cfg, tensor_id, shape, std=1.0, mean=0.0, row0=0, nrows=None):
    """float32 N(mean, std^2); ``shape`` = (..., cols); rows = prod(leading dims)."""
    cols = shape[-1]
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    if nrows is None:
        nrows = rows - row0
        out_shape = shape
    else:
        out_shape = (nrows, cols)
    return _draw_rows(cfg, tensor_id, row0, nrows, cols, "normal", mean, std).reshape(out_shape)


def uniform_f32(cfg, tensor_id, shape, lo=0.0, hi=1.0):
    cols = shape[-1]
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    return _draw_rows(cfg, tensor_id, 0, rows, cols, "uniform", lo, hi).reshape(shape)


def normal_bf16(cfg, tensor_id, shape, std=1.0, mean=0.0, row0=0, nrows=None):
    """bf16 bit patterns (uint16) of seeded N(mean, std^2) draws."""
    return f32_to_bf16_bits(normal_f32(cfg, tensor_id, shape, std, mean, row0, nrows))


# ---------------------------------------------------------------------------------------------
# Workload descriptions.  Sizes follow the five workloads of the hybrid-attention pages:
# the CSA ratio m = 4 with overlap, HCA ratio m' = 128, top-k 1024, window 128, shared-KV
# head dim 512 with 64 query heads and 64-dim partial RoPE, indexer 64 heads x 128.
# ---------------------------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg: int                 # seed id
    kind: str                # "csa_forward" | "csa_decode" | "csa_prefill" | "hca_decode"
    B: int
    T: int                   # context tokens per sequence (decode: query at t = T - 1)
    d: int                   # shared KV dim (= query head dim D)
    H: int                   # query heads
    rope_dim: int
    m: int
    overlap: int
    H_I: int = 0
    D_I: int = 0
    key_format: str = "none"  # "f32" | "fp8" | "mxfp4"
    topk: int = 0
    window: int = 128
    Sq: int = 1               # query tokens per sequence
    n_planted: int = 0
    bias_std: float = 0.1
    w_dist: str = "uniform"   # indexer head weights: "uniform" U(0,1) or "normal" N(0,1)

    @property
    def N(self) -> int:
        return self.T // self.m

    @property
    def rows_per_query(self) -> int:
        if self.kind == "hca_decode":
            return self.N + self.window
        return self.topk + self.window


TINY = Workload("csa_forward_tiny_256", 0, "csa_forward", B=1, T=256, d=64, H=8, rope_dim=16, m=4,
                overlap=1, H_I=4, D_I=32, key_format="f32", topk=16, window=32, Sq=256,
                w_dist="normal")
CSA_DECODE_32K = Workload("csa_decode_32k_b16_fp8", 1, "csa_decode", B=16, T=32768, d=512, H=64,
                          rope_dim=64, m=4, overlap=1, H_I=64, D_I=128, key_format="fp8", topk=1024)
CSA_PREFILL_128K = Workload("csa_prefill_4096_at_128k_fp8", 2, "csa_prefill", B=1, T=131072, d=512,
                            H=64, rope_dim=64, m=4, overlap=1, H_I=64, D_I=128, key_format="fp8",
                            topk=1024, Sq=4096)
HCA_DECODE_1M = Workload("hca_decode_1m_b8", 3, "hca_decode", B=8, T=1048576, d=512, H=64,
                         rope_dim=64, m=128, overlap=0)
CSA_DECODE_1M = Workload("csa_decode_1m_b4_mxfp4", 4, "csa_decode", B=4, T=1048576, d=512, H=64,
                         rope_dim=64, m=4, overlap=1, H_I=64, D_I=128, key_format="mxfp4",
                         topk=1024, n_planted=16)
# The Flash configuration's attention top-k (512) at the maximum context, else as above.
CSA_DECODE_1M_FLASH = Workload("csa_decode_1m_b4_mxfp4_k512", 4, "csa_decode", B=4, T=1048576, d=512, H=64,
                               rope_dim=64, m=4, overlap=1, H_I=64, D_I=128, key_format="mxfp4",
                               topk=512, n_planted=16)
# Derived decode point at 128K context with the 32K decode shapes (the metric names 128K decode).
CSA_DECODE_128K = Workload("csa_decode_128k_b16_fp8", 5, "csa_decode", B=16, T=131072, d=512, H=64,
                           rope_dim=64, m=4, overlap=1, H_I=64, D_I=128, key_format="fp8", topk=1024)

WORKLOADS = {w.name: w for w in (TINY, CSA_DECODE_32K, CSA_PREFILL_128K, HCA_DECODE_1M,
                                 CSA_DECODE_1M, CSA_DECODE_128K, CSA_DECODE_1M_FLASH)}


def decode_inputs(w: Workload, b_lo: int = 0, b_hi: int | None = None, n_rows: int | None = None,
                  parts=("attend", "index")):
    """Host-side decode inputs for sequences [b_lo, b_hi).

    Returns a dict of numpy arrays: bf16 tensors as uint16 bit patterns, fp32 otherwise.
    ``n_rows`` limits the entries/keys to the first n rows (for sampled checks); the planted
    entries are placed relative to the full N.  ``parts`` selects the attention inputs (q,
    entries, window rows) and/or the indexer inputs (q_idx, w_idx, k_idx).
    """
    b_hi = w.B if b_hi is None else b_hi
    nb = b_hi - b_lo
    N = w.N if n_rows is None else n_rows
    d, H = w.d, w.H
    out = {}
    if "attend" in parts:
        out["q"] = normal_bf16(w.cfg, T_Q, (w.B * w.Sq * H, d), row0=b_lo * w.Sq * H,
                               nrows=nb * w.Sq * H).reshape(nb, w.Sq, H, d)
        out["win_rows"] = normal_bf16(w.cfg, T_WIN, (w.B * w.window, d), row0=b_lo * w.window,
                                      nrows=nb * w.window).reshape(nb, w.window, d)
        ent = np.empty((nb, N, d), dtype=np.uint16)
        for j, b in enumerate(range(b_lo, b_hi)):
            ent[j] = normal_bf16(w.cfg, T_ENTRIES, (w.B * w.N, d), row0=b * w.N, nrows=N)
        out["entries"] = ent
    if w.kind == "csa_decode" and "index" in parts:
        out["q_idx"] = normal_bf16(w.cfg, T_QIDX, (w.B * w.Sq * w.H_I, w.D_I), row0=b_lo * w.Sq * w.H_I,
                                   nrows=nb * w.Sq * w.H_I).reshape(nb, w.Sq, w.H_I, w.D_I)
        wts = uniform_f32(w.cfg, T_W, (w.B * w.Sq, w.H_I))
        out["w_idx"] = wts[b_lo * w.Sq:b_hi * w.Sq].reshape(nb, w.Sq, w.H_I)
        kf = np.empty((nb, N, w.D_I), dtype=np.float32)
        for j, b in enumerate(range(b_lo, b_hi)):
            kf[j] = normal_f32(w.cfg, T_KIDX, (w.B * w.N, w.D_I), row0=b * w.N, nrows=N)
        if w.n_planted:
            planted = planted_indices(w)
            for j, b in enumerate(range(b_lo, b_hi)):
                kp = planted_key(out["q_idx"][j, 0], out["w_idx"][j, 0])
                for i in planted[b]:
                    if i < N:
                        kf[j, i] = kp
        out["k_idx"] = f32_to_bf16_bits(kf)
    out["t"] = np.full((nb,), w.T - 1, dtype=np.int64)
    out["win_pos0"] = np.full((nb,), w.T - w.window, dtype=np.int64)
    out["n_entries"] = np.full((nb,), w.N, dtype=np.int64)
    return out


def planted_indices(w: Workload) -> list[np.ndarray]:
    """Per sequence: ``n_planted`` distinct entry indices, always including 0 and N-1."""
    res = []
    for b in range(w.B):
        g = _rng(w.cfg, T_PLANT, b)
        others = g.choice(np.arange(1, w.N - 1), size=w.n_planted - 2, replace=False)
        res.append(np.sort(np.concatenate([[0, w.N - 1], others])).astype(np.int64))
    return res


def planted_key(q_idx_bf16: np.ndarray, w_row: np.ndarray) -> np.ndarray:
    """Key for a planted entry: a scaled copy of the weighted query, 4*sqrt(D_I)*qbar/|qbar|."""
    q = bf16_bits_to_f32(q_idx_bf16).astype(np.float64)      # [H_I, D_I]
    qbar = (w_row.astype(np.float64)[:, None] * q).sum(0)
    return (4.0 * math.sqrt(q.shape[1]) * qbar / np.linalg.norm(qbar)).astype(np.float32)


def tiny_inputs(w: Workload = TINY):
    """The tiny single-layer CSA forward: token stream, compressor parameters, queries, indexer."""
    T, d = w.T, w.d
    return {
        "c": normal_bf16(w.cfg, T_C, (T, d)).reshape(1, T, d),
        "z": normal_bf16(w.cfg, T_Z, (T, d)).reshape(1, T, d),
        "bias": normal_bf16(w.cfg, T_BIAS, ((1 + w.overlap) * w.m, d), std=w.bias_std),
        "q": normal_bf16(w.cfg, T_Q, (T * w.H, d)).reshape(1, T, w.H, d),
        "q_idx": normal_f32(w.cfg, T_QIDX, (T * w.H_I, w.D_I)).reshape(1, T, w.H_I, w.D_I),
        "w_idx": normal_f32(w.cfg, T_W, (T, w.H_I)).reshape(1, T, w.H_I),
        "k_idx": normal_f32(w.cfg, T_KIDX, (w.N, w.D_I)).reshape(1, w.N, w.D_I),
    }
