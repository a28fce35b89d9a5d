"""Python binding of libcsa: argument marshalling only.

Each function takes torch tensors that already live on the GPU, checks dtype/shape/contiguity,
allocates outputs and workspace with torch (device memory is plumbing), and calls the C-ABI
function of the same name on the current torch stream.  Every step of the computation runs in the
HIP library; there is no fallback: if ``libcsa.so`` is missing the first call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa.so")

KEY_F32, KEY_FP8_E4M3, KEY_MXFP4 = 0, 1, 2
KEY_FORMATS = {"f32": KEY_F32, "fp8": KEY_FP8_E4M3, "mxfp4": KEY_MXFP4}
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace", 4: "HIP error"}

_lib = None
P = ctypes.c_void_p
I32, I64, F32, SZ = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t

_SIGS = {
    "csa_compress": (I32, [P, P, P, P, I32, I64, I32, I32, I32, I32, I32, I64, F32, F32, P, P, P]),
    "csa_quantize_keys": (I32, [P, I64, I32, I32, P, P, P]),
    "csa_quantize_query": (I32, [P, P, I64, I32, I32, P, P, P, P]),
    "csa_output_projection": (I32, [P, P, I32, I32, I32, I32, I32, P, P]),
    "csa_compress_index_keys": (I32, [P, P, P, I32, I64, I32, I32, I32, I32, I64, I32, P, P, P, P]),
    "csa_decode_append_index": (I32, [P, P, P, P, I32, I32, I32, I32, P, P, I64, I32, P, P, P, P]),
    "csa_decode_append_step": (I32, [P, P, P, P, P, I32, I32, I32, I32, I32, F32, F32, P, P, P, I64, P, I64, P,
                                     P, P, P, I32, P, P, I32, P, P, P, P]),
    "csa_decode_append": (I32, [P, P, P, P, P, P, I32, I32, I32, I32, I32, F32, F32, P, P, P, I64, P, I64,
                                I32, I32, P, P, P, P]),
    "csa_index_topk": (I32, [P, P, P, P, I32, I32, I32, I32, I32, I64, P, P, I32, I32, P, P, P, SZ, P]),
    "csa_index_topk_workspace_bytes": (SZ, [I32, I32, I64, I32]),
    "csa_attend": (I32, [P, P, P, I64, P, I32, P, I64, P, P, I32, I32, I32, I32, I32, I32, F32, F32,
                         F32, P, P, P, SZ, P]),
    "csa_attend_workspace_bytes": (SZ, [I32, I32, I32, I32, I32, I32]),
    "csa_attend_noalloc": (I32, [P, P, P, I64, P, I32, P, I64, P, P, I32, I32, I32, I32, I32, I32, F32, F32,
                                 F32, P, P, P]),
    "hca_attend": (I32, [P, P, P, I64, P, I32, P, I64, P, P, I32, I32, I32, I32, I32, I32, F32, F32,
                         F32, P, P, P, SZ, P]),
    "hca_attend_workspace_bytes": (SZ, [I32, I32, I32, I32, I64, I32]),
    "csa_status_string": (ctypes.c_char_p, [I32]),
    "csa_last_error": (ctypes.c_char_p, []),
    "csa_timing_enable": (None, [I32]),
    "csa_measure_stream_read": (I32, [P, I64, P, P]),
    "csa_timing_read": (I32, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64)]),
}


class CsaError(RuntimeError):
    pass


def lib():
    """Load libcsa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise CsaError(f"{LIB_PATH} is missing: build it with "
                           "`python -m compressed_sparse_attention_03_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != 0:
        detail = lib().csa_last_error().decode()
        raise CsaError(f"{what}: {STATUS.get(status, status)}: {detail}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, name, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _i64(t, name, B):
    t = _dev(t, name, torch.int64, 1)
    if t.shape[0] != B:
        raise ValueError(f"{name} must have shape [{B}]")
    return t


# ---------------------------------------------------------------------------------------------
def csa_compress(c, z, bias, *, m, overlap, rope_dim, pos0=0, norm_w=None, rope_base=10000.0,
                 eps=1e-6, win_rows=False, entries_out=None, win_rows_out=None):
    """Compressed entries [B, n_new/m, d] (and prepared window rows [B, n_new, d] if asked)."""
    _dev(c, "c", torch.bfloat16, 3)
    _dev(z, "z", torch.bfloat16, 3)
    _dev(bias, "bias", torch.bfloat16, 2)
    B, rows, d = c.shape
    if z.shape != c.shape:
        raise ValueError("z must have the shape of c")
    halo = m if (overlap and pos0 > 0) else 0
    n_new = rows - halo
    ent = entries_out if entries_out is not None else torch.empty((B, max(n_new, 0) // m, d), dtype=torch.bfloat16, device=c.device)
    wr = None
    if win_rows:
        wr = win_rows_out if win_rows_out is not None else torch.empty((B, n_new, d), dtype=torch.bfloat16, device=c.device)
    if norm_w is not None:
        _dev(norm_w, "norm_w", torch.bfloat16, 1)
    st = lib().csa_compress(_ptr(c), _ptr(z), _ptr(bias), _ptr(norm_w), B, n_new, halo, d, m, overlap,
                            rope_dim, pos0, rope_base, eps, _ptr(ent), _ptr(wr), _stream())
    _check(st, "csa_compress")
    return ent, wr


def csa_quantize_keys(x, fmt, codes_out=None, scales_out=None):
    """Keys bf16 [..., dim] -> (codes, scales) in the storage format ``fmt`` ("fp8" | "mxfp4").
    ``codes_out`` / ``scales_out`` (contiguous, of the output shapes) receive the result in place."""
    _dev(x, "x", torch.bfloat16)
    dim = x.shape[-1]
    rows = x.numel() // dim
    f = KEY_FORMATS[fmt]
    lead = tuple(x.shape[:-1])
    if f == KEY_FP8_E4M3:
        cshape, sshape, sdtype = lead + (dim,), lead, torch.float32
    else:
        cshape, sshape, sdtype = lead + (dim // 2,), lead + (dim // 32,), torch.uint8
    codes = codes_out if codes_out is not None else torch.empty(cshape, dtype=torch.uint8, device=x.device)
    scales = scales_out if scales_out is not None else torch.empty(sshape, dtype=sdtype, device=x.device)
    _dev(codes, "codes_out", torch.uint8)
    _dev(scales, "scales_out", sdtype)
    if tuple(codes.shape) != cshape or tuple(scales.shape) != sshape:
        raise ValueError(f"outputs must have shapes {cshape} and {sshape}")
    st = lib().csa_quantize_keys(_ptr(x), rows, dim, f, _ptr(codes), _ptr(scales), _stream())
    _check(st, "csa_quantize_keys")
    return codes, scales


def csa_quantize_query(q_idx, w_idx, fmt):
    """The indexer's query encoding: q_idx bf16 [..., H_I, 128], w_idx fp32 [..., H_I] ->
    (codes uint8 [..., H_I, 128 | 64], scale bytes uint8 [..., H_I, 4] or None, factors fp32 [..., H_I])."""
    _dev(q_idx, "q_idx", torch.bfloat16)
    _dev(w_idx, "w_idx", torch.float32)
    H_I = q_idx.shape[-2]
    if q_idx.shape[-1] != 128 or tuple(w_idx.shape) != tuple(q_idx.shape[:-1]):
        raise ValueError("q_idx must be [..., H_I, 128] and w_idx [..., H_I]")
    lead = tuple(q_idx.shape[:-2])
    n = q_idx.numel() // (H_I * 128)
    f = KEY_FORMATS[fmt]
    codes = torch.empty(lead + (H_I, 128 if f == KEY_FP8_E4M3 else 64), dtype=torch.uint8, device=q_idx.device)
    sb = torch.empty(lead + (H_I, 4), dtype=torch.uint8, device=q_idx.device) if f == KEY_MXFP4 else None
    factors = torch.empty(lead + (H_I,), dtype=torch.float32, device=q_idx.device)
    st = lib().csa_quantize_query(_ptr(q_idx), _ptr(w_idx), n, H_I, f, _ptr(codes), _ptr(sb), _ptr(factors),
                                  _stream())
    _check(st, "csa_quantize_query")
    return codes, sb, factors


def _key_cache_shapes(lead, D_I, f):
    if f == KEY_F32:
        return (lead + (D_I,), torch.float32), None
    if f == KEY_FP8_E4M3:
        return (lead + (D_I,), torch.uint8), (lead, torch.float32)
    return (lead + (D_I // 2,), torch.uint8), (lead + (D_I // 32,), torch.uint8)


def _check_key_cache(k_codes, k_scales, lead, D_I, f):
    cs, ss = _key_cache_shapes(lead, D_I, f)
    _dev(k_codes, "k_codes", cs[1])
    if tuple(k_codes.shape) != cs[0]:
        raise ValueError(f"k_codes must have shape {cs[0]}")
    if ss is not None:
        _dev(k_scales, "k_scales", ss[1])
        if tuple(k_scales.shape) != ss[0]:
            raise ValueError(f"k_scales must have shape {ss[0]}")


def csa_compress_index_keys(c_i, z_i, bias_i, *, m, overlap, key_format, pos0=0, keys_out=False,
                            k_codes=None, k_scales=None):
    """Indexer keys by compression of the per-token stream c_i/z_i [B, halo+n_new, D_I]:
    (codes, scales, bf16 keys or None) for entries pos0/m .. in ``key_format``."""
    _dev(c_i, "c_i", torch.bfloat16, 3)
    _dev(z_i, "z_i", torch.bfloat16, 3)
    _dev(bias_i, "bias_i", torch.bfloat16, 2)
    B, rows, D_I = c_i.shape
    if z_i.shape != c_i.shape:
        raise ValueError("z_i must have the shape of c_i")
    halo = m if (overlap and pos0 > 0) else 0
    n_new = rows - halo
    n_out = max(n_new, 0) // m
    f = KEY_FORMATS[key_format]
    cs, ss = _key_cache_shapes((B, n_out), D_I, f)
    codes = k_codes if k_codes is not None else torch.empty(cs[0], dtype=cs[1], device=c_i.device)
    scales = None
    if ss is not None:
        scales = k_scales if k_scales is not None else torch.empty(ss[0], dtype=ss[1], device=c_i.device)
    _check_key_cache(codes, scales, (B, n_out), D_I, f)
    ko = torch.empty((B, n_out, D_I), dtype=torch.bfloat16, device=c_i.device) if keys_out else None
    st = lib().csa_compress_index_keys(_ptr(c_i), _ptr(z_i), _ptr(bias_i), B, n_new, halo, D_I, m, overlap, pos0,
                                       f, _ptr(ko), _ptr(codes), _ptr(scales), _stream())
    _check(st, "csa_compress_index_keys")
    return codes, scales, ko


def csa_decode_append_index(c_i_new, z_i_new, pos, bias_i, *, m, overlap, tok_c, tok_z, key_format, k_codes,
                            k_scales=None, keys_out=None):
    """The indexer stream's decode-time maintenance, in place: ring ``tok_c``/``tok_z``
    [B, (1+overlap)*m, D_I] and key cache ``k_codes``/``k_scales`` ([B, N_cap] rows)."""
    _dev(c_i_new, "c_i_new", torch.bfloat16, 2)
    _dev(z_i_new, "z_i_new", torch.bfloat16, 2)
    B, D_I = c_i_new.shape
    if tuple(z_i_new.shape) != (B, D_I):
        raise ValueError("z_i_new must have the shape of c_i_new")
    _i64(pos, "pos", B)
    _dev(bias_i, "bias_i", torch.bfloat16, 2)
    R = (1 + overlap) * m
    for name, t in (("tok_c", tok_c), ("tok_z", tok_z)):
        _dev(t, name, torch.bfloat16, 3)
        if tuple(t.shape) != (B, R, D_I):
            raise ValueError(f"{name} must be [{B}, {R}, {D_I}]")
    f = KEY_FORMATS[key_format]
    N_cap = k_codes.shape[1]
    _check_key_cache(k_codes, k_scales, (B, N_cap), D_I, f)
    if keys_out is not None:
        _dev(keys_out, "keys_out", torch.bfloat16, 3)
        if tuple(keys_out.shape) != (B, N_cap, D_I):
            raise ValueError(f"keys_out must be [{B}, {N_cap}, {D_I}]")
    st = lib().csa_decode_append_index(_ptr(c_i_new), _ptr(z_i_new), _ptr(pos), _ptr(bias_i), B, D_I, m, overlap,
                                       _ptr(tok_c), _ptr(tok_z), N_cap, f, _ptr(keys_out), _ptr(k_codes),
                                       _ptr(k_scales), _stream())
    _check(st, "csa_decode_append_index")


def csa_decode_append(c_new, z_new, pos, bias, *, m, overlap, rope_dim, tok_c, tok_z, win_ring, entries,
                      n_entries, k_new=None, key_format="fp8", k_codes=None, k_scales=None, norm_w=None,
                      rope_base=10000.0, eps=1e-6):
    """Decode-time cache maintenance for one new token per sequence, in place on the caches:
    token ring ``tok_c``/``tok_z`` [B, (1+overlap)*m, d], window ring ``win_ring`` [B, W_cap, d],
    ``entries`` [B, N_cap, d], indexer keys ``k_codes``/``k_scales`` and ``n_entries`` [B]."""
    _dev(c_new, "c_new", torch.bfloat16, 2)
    _dev(z_new, "z_new", torch.bfloat16, 2)
    B, d = c_new.shape
    if tuple(z_new.shape) != (B, d):
        raise ValueError("z_new must have the shape of c_new")
    _i64(pos, "pos", B)
    _i64(n_entries, "n_entries", B)
    _dev(bias, "bias", torch.bfloat16, 2)
    R = (1 + overlap) * m
    for name, t in (("tok_c", tok_c), ("tok_z", tok_z)):
        _dev(t, name, torch.bfloat16, 3)
        if tuple(t.shape) != (B, R, d):
            raise ValueError(f"{name} must be [{B}, {R}, {d}]")
    _dev(win_ring, "win_ring", torch.bfloat16, 3)
    _dev(entries, "entries", torch.bfloat16, 3)
    if win_ring.shape[0] != B or win_ring.shape[2] != d or entries.shape[0] != B or entries.shape[2] != d:
        raise ValueError("win_ring / entries must be [B, rows, d]")
    if norm_w is not None:
        _dev(norm_w, "norm_w", torch.bfloat16, 1)
    N_cap = entries.shape[1]
    f, D_I = KEY_FORMATS[key_format], 0
    if k_new is not None:
        _dev(k_new, "k_new", torch.bfloat16, 2)
        D_I = k_new.shape[1]
        if k_new.shape[0] != B:
            raise ValueError("k_new must be [B, D_I]")
        if f == KEY_F32:
            shapes = {"k_codes": ((B, N_cap, D_I), torch.float32)}
        elif f == KEY_FP8_E4M3:
            shapes = {"k_codes": ((B, N_cap, D_I), torch.uint8), "k_scales": ((B, N_cap), torch.float32)}
        else:
            shapes = {"k_codes": ((B, N_cap, D_I // 2), torch.uint8),
                      "k_scales": ((B, N_cap, D_I // 32), torch.uint8)}
        for name, t in (("k_codes", k_codes), ("k_scales", k_scales)):
            if name in shapes:
                shp, dt = shapes[name]
                _dev(t, name, dt)
                if tuple(t.shape) != shp:
                    raise ValueError(f"{name} must have shape {shp}")
    st = lib().csa_decode_append(_ptr(c_new), _ptr(z_new), _ptr(k_new), _ptr(pos), _ptr(bias), _ptr(norm_w), B, d,
                                 m, overlap, rope_dim, rope_base, eps, _ptr(tok_c), _ptr(tok_z), _ptr(win_ring),
                                 win_ring.shape[1], _ptr(entries), N_cap, f, D_I, _ptr(k_codes), _ptr(k_scales),
                                 _ptr(n_entries), _stream())
    _check(st, "csa_decode_append")


def csa_decode_append_step(c_new, z_new, pos, bias, *, m, overlap, rope_dim, tok_c, tok_z, win_ring, entries,
                           n_entries, c_i_new, z_i_new, bias_i, tok_ci, tok_zi, key_format, k_codes, k_scales=None,
                           keys_out=None, norm_w=None, rope_base=10000.0, eps=1e-6):
    """A decode step's whole cache maintenance in one launch: csa_decode_append's KV stream
    (without k_new) and csa_decode_append_index's indexer stream, in place on the caches."""
    _dev(c_new, "c_new", torch.bfloat16, 2)
    _dev(z_new, "z_new", torch.bfloat16, 2)
    B, d = c_new.shape
    if tuple(z_new.shape) != (B, d):
        raise ValueError("z_new must have the shape of c_new")
    _i64(pos, "pos", B)
    _i64(n_entries, "n_entries", B)
    _dev(bias, "bias", torch.bfloat16, 2)
    R = (1 + overlap) * m
    for name, t in (("tok_c", tok_c), ("tok_z", tok_z)):
        _dev(t, name, torch.bfloat16, 3)
        if tuple(t.shape) != (B, R, d):
            raise ValueError(f"{name} must be [{B}, {R}, {d}]")
    _dev(win_ring, "win_ring", torch.bfloat16, 3)
    _dev(entries, "entries", torch.bfloat16, 3)
    if win_ring.shape[0] != B or win_ring.shape[2] != d or entries.shape[0] != B or entries.shape[2] != d:
        raise ValueError("win_ring / entries must be [B, rows, d]")
    if norm_w is not None:
        _dev(norm_w, "norm_w", torch.bfloat16, 1)
    N_cap = entries.shape[1]
    _dev(c_i_new, "c_i_new", torch.bfloat16, 2)
    _dev(z_i_new, "z_i_new", torch.bfloat16, 2)
    D_I = c_i_new.shape[1]
    if c_i_new.shape[0] != B or tuple(z_i_new.shape) != (B, D_I):
        raise ValueError("c_i_new / z_i_new must be [B, D_I]")
    _dev(bias_i, "bias_i", torch.bfloat16, 2)
    for name, t in (("tok_ci", tok_ci), ("tok_zi", tok_zi)):
        _dev(t, name, torch.bfloat16, 3)
        if tuple(t.shape) != (B, R, D_I):
            raise ValueError(f"{name} must be [{B}, {R}, {D_I}]")
    f = KEY_FORMATS[key_format]
    if k_codes.shape[1] != N_cap:
        raise ValueError("k_codes must have N_cap rows per sequence, as entries")
    _check_key_cache(k_codes, k_scales, (B, N_cap), D_I, f)
    if keys_out is not None:
        _dev(keys_out, "keys_out", torch.bfloat16, 3)
        if tuple(keys_out.shape) != (B, N_cap, D_I):
            raise ValueError(f"keys_out must be [{B}, {N_cap}, {D_I}]")
    st = lib().csa_decode_append_step(_ptr(c_new), _ptr(z_new), _ptr(pos), _ptr(bias), _ptr(norm_w), B, d, m, overlap,
                                      rope_dim, rope_base, eps, _ptr(tok_c), _ptr(tok_z), _ptr(win_ring),
                                      win_ring.shape[1], _ptr(entries), N_cap, _ptr(n_entries), _ptr(c_i_new),
                                      _ptr(z_i_new), _ptr(bias_i), D_I, _ptr(tok_ci), _ptr(tok_zi), f, _ptr(keys_out),
                                      _ptr(k_codes), _ptr(k_scales), _stream())
    _check(st, "csa_decode_append_step")


def index_topk_workspace(B, Sq, N_cap, topk, device="cuda"):
    n = lib().csa_index_topk_workspace_bytes(B, Sq, N_cap, topk)
    return torch.zeros(n, dtype=torch.uint8, device=device)     # zero once: it holds counters


def csa_index_topk(q_idx, w_idx, k_codes, k_scales, *, key_format, n_entries, q_pos0, m, topk,
                   scores=False, workspace=None, topk_out=None):
    """Top-k entry indices int32 [B, Sq, topk] (ascending, -1 padded) and optionally the scores."""
    f = KEY_FORMATS[key_format] if isinstance(key_format, str) else int(key_format)
    _dev(q_idx, "q_idx", torch.float32 if f == KEY_F32 else torch.bfloat16, 4)
    B, Sq, H_I, D_I = q_idx.shape
    _dev(w_idx, "w_idx", torch.float32, 3)
    if tuple(w_idx.shape) != (B, Sq, H_I):
        raise ValueError("w_idx must be [B, Sq, H_I]")
    _dev(k_codes, "k_codes", torch.float32 if f == KEY_F32 else torch.uint8, 3)
    N_cap = k_codes.shape[1]
    if k_codes.shape[0] != B:
        raise ValueError("k_codes must be [B, N_cap, ...]")
    if f != KEY_F32:
        _dev(k_scales, "k_scales")
    _i64(n_entries, "n_entries", B)
    _i64(q_pos0, "q_pos0", B)
    out = topk_out if topk_out is not None else torch.empty((B, Sq, topk), dtype=torch.int32, device=q_idx.device)
    sc = torch.empty((B, Sq, N_cap), dtype=torch.float32, device=q_idx.device) if scores else None
    ws = workspace if workspace is not None else index_topk_workspace(B, Sq, N_cap, topk, q_idx.device)
    st = lib().csa_index_topk(_ptr(q_idx), _ptr(w_idx), _ptr(k_codes), _ptr(k_scales), f, B, Sq, H_I, D_I,
                              N_cap, _ptr(n_entries), _ptr(q_pos0), m, topk, _ptr(out), _ptr(sc),
                              _ptr(ws), ws.numel(), _stream())
    _check(st, "csa_index_topk")
    return out, sc


def attend_workspace(B, Sq, H, D, topk, window, device="cuda"):
    n = lib().csa_attend_workspace_bytes(B, Sq, H, D, topk, window)
    return torch.zeros(n, dtype=torch.uint8, device=device)     # zero once: it holds counters


def hca_workspace(B, Sq, H, D, N_cap, window, device="cuda"):
    n = lib().hca_attend_workspace_bytes(B, Sq, H, D, N_cap, window)
    return torch.zeros(n, dtype=torch.uint8, device=device)     # zero once: it holds counters


def _attend_common(q, entries, win_rows, win_pos0, q_pos0, q_norm_w):
    _dev(q, "q", torch.bfloat16, 4)
    B, Sq, H, D = q.shape
    _dev(entries, "entries", torch.bfloat16, 3)
    _dev(win_rows, "win_rows", torch.bfloat16, 3)
    if entries.shape[0] != B or entries.shape[2] != D or win_rows.shape[0] != B or win_rows.shape[2] != D:
        raise ValueError("entries/win_rows must be [B, rows, D]")
    if win_pos0 is not None:                     # None: win_rows is a ring (row p mod W_cap)
        _i64(win_pos0, "win_pos0", B)
    _i64(q_pos0, "q_pos0", B)
    if q_norm_w is not None:
        _dev(q_norm_w, "q_norm_w", torch.bfloat16, 1)
    return B, Sq, H, D


def csa_attend(q, entries, topk_idx, win_rows, win_pos0, q_pos0, *, rope_dim, window, q_norm_w=None,
               softmax_scale=None, rope_base=10000.0, eps=1e-6, lse=False, workspace=None, out=None):
    """CSA core attention -> (out bf16 [B, Sq, H, D], lse fp32 [B, Sq, H] or None)."""
    B, Sq, H, D = _attend_common(q, entries, win_rows, win_pos0, q_pos0, q_norm_w)
    _dev(topk_idx, "topk_idx", torch.int32, 3)
    topk = topk_idx.shape[2]
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else softmax_scale
    o = out if out is not None else torch.empty_like(q)
    ls = torch.empty((B, Sq, H), dtype=torch.float32, device=q.device) if lse else None
    ws = workspace if workspace is not None else attend_workspace(B, Sq, H, D, topk, window, q.device)
    st = lib().csa_attend(_ptr(q), _ptr(q_norm_w), _ptr(entries), entries.shape[1], _ptr(topk_idx), topk,
                          _ptr(win_rows), win_rows.shape[1], _ptr(win_pos0), _ptr(q_pos0), B, Sq, H, D,
                          rope_dim, window, scale, rope_base, eps, _ptr(o), _ptr(ls), _ptr(ws), ws.numel(),
                          _stream())
    _check(st, "csa_attend")
    return o, ls


def csa_attend_noalloc(q, entries, topk_idx, win_rows, win_pos0, q_pos0, *, rope_dim, window, q_norm_w=None,
                       softmax_scale=None, rope_base=10000.0, eps=1e-6, out, lse=None):
    """csa_attend with the library's own scratch (no workspace): ``out`` (and ``lse`` if wanted)
    must be given, so the call itself allocates nothing."""
    B, Sq, H, D = _attend_common(q, entries, win_rows, win_pos0, q_pos0, q_norm_w)
    _dev(topk_idx, "topk_idx", torch.int32, 3)
    _dev(out, "out", torch.bfloat16, 4)
    if tuple(out.shape) != (B, Sq, H, D) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, Sq, H, D] tensor")
    if lse is not None:
        _dev(lse, "lse", torch.float32, 3)
        if tuple(lse.shape) != (B, Sq, H) or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous [B, Sq, H] tensor")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else softmax_scale
    st = lib().csa_attend_noalloc(_ptr(q), _ptr(q_norm_w), _ptr(entries), entries.shape[1], _ptr(topk_idx),
                                  topk_idx.shape[2], _ptr(win_rows), win_rows.shape[1], _ptr(win_pos0), _ptr(q_pos0),
                                  B, Sq, H, D, rope_dim, window, scale, rope_base, eps, _ptr(out), _ptr(lse),
                                  _stream())
    _check(st, "csa_attend_noalloc")
    return out, lse


def hca_attend(q, entries, n_entries, win_rows, win_pos0, q_pos0, *, m, rope_dim, window, q_norm_w=None,
               softmax_scale=None, rope_base=10000.0, eps=1e-6, lse=False, workspace=None, out=None):
    """HCA core attention (dense over visible entries + window) -> (out, lse or None)."""
    B, Sq, H, D = _attend_common(q, entries, win_rows, win_pos0, q_pos0, q_norm_w)
    _i64(n_entries, "n_entries", B)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else softmax_scale
    o = out if out is not None else torch.empty_like(q)
    ls = torch.empty((B, Sq, H), dtype=torch.float32, device=q.device) if lse else None
    N_cap = entries.shape[1]
    ws = workspace if workspace is not None else hca_workspace(B, Sq, H, D, N_cap, window, q.device)
    st = lib().hca_attend(_ptr(q), _ptr(q_norm_w), _ptr(entries), N_cap, _ptr(n_entries), m, _ptr(win_rows),
                          win_rows.shape[1], _ptr(win_pos0), _ptr(q_pos0), B, Sq, H, D, rope_dim, window,
                          scale, rope_base, eps, _ptr(o), _ptr(ls), _ptr(ws), ws.numel(), _stream())
    _check(st, "hca_attend")
    return o, ls


def csa_output_projection(o, w, out=None):
    """Grouped output projection: o bf16 [..., H, D] (heads last) and w bf16 [G, N_g, H*D/G] ->
    y bf16 [..., G*N_g]."""
    _dev(o, "o", torch.bfloat16)
    _dev(w, "w", torch.bfloat16, 3)
    H, D = o.shape[-2], o.shape[-1]
    M = o.numel() // (H * D)
    G, N_g, K_g = w.shape
    if G * K_g != H * D:
        raise ValueError("w must be [G, N_g, H*D/G]")
    y = out if out is not None else torch.empty(tuple(o.shape[:-2]) + (G * N_g,), dtype=torch.bfloat16, device=o.device)
    _dev(y, "out", torch.bfloat16)
    if y.numel() != M * G * N_g:
        raise ValueError("out must hold [..., G*N_g]")
    st = lib().csa_output_projection(_ptr(o), _ptr(w), M, H, D, G, N_g, _ptr(y), _stream())
    _check(st, "csa_output_projection")
    return y


def timing_enable(on: bool):
    lib().csa_timing_enable(1 if on else 0)


def measure_stream_read(src, sink):
    """Plain streaming read of every byte of ``src`` (a CUDA tensor of a multiple of 16 bytes);
    ``sink`` is a CUDA tensor of at least 4 bytes that the read may write."""
    if not (isinstance(src, torch.Tensor) and src.is_cuda and src.is_contiguous()):
        raise TypeError("src must be a contiguous CUDA (HIP) tensor")
    if not (isinstance(sink, torch.Tensor) and sink.is_cuda and sink.numel() * sink.element_size() >= 4):
        raise TypeError("sink must be a CUDA (HIP) tensor of at least 4 bytes")
    _check(lib().csa_measure_stream_read(ctypes.c_void_p(src.data_ptr()), src.numel() * src.element_size(),
                                         ctypes.c_void_p(sink.data_ptr()), _stream()), "csa_measure_stream_read")


def timing_read(kernel: str):
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib().csa_timing_read(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)), "csa_timing_read")
    return ms.value, n.value
