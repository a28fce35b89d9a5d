"""Shared helpers of the GPU parity tests: host<->device conversion and the comparison rules.

Tolerances (bf16 I/O, fp32 accumulation): compressed entries and attention outputs within
max-abs 2e-2 and mean-abs 2e-3; indexer scores within 1e-2 relative (plus 1e-4 of the row's
largest magnitude); top-k sets equal except for entries whose score lies within 1e-3 (absolute)
of the k-th score (those near-ties may legitimately differ between a float32 and a float64
evaluation).
"""
import sys

import numpy as np
import torch

from compressed_sparse_attention_03_amd.inputs import bf16_bits_to_f32

MAX_ABS, MEAN_ABS = 2e-2, 2e-3
SCORE_REL, SCORE_FLOOR = 1e-2, 1e-4
TIE_ABS = 1e-3          # set differences allowed only within this distance of the k-th score


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


def dev(x: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def f64(u16: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(u16).astype(np.float64)


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU values"
    err = np.abs(gpu - ref)
    mx, mean = float(err.max()), float(err.mean())
    rel = float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-30))
    say(f"  {what}: max_abs={mx:.3e} mean_abs={mean:.3e} rel_l2={rel:.3e}")
    assert mx <= max_abs and mean <= mean_abs, f"{what}: max_abs {mx} mean_abs {mean}"


def assert_scores(gpu: np.ndarray, ref: np.ndarray, what: str):
    vis = np.isfinite(ref)
    assert (np.isneginf(gpu[~vis])).all(), f"{what}: invisible entries must be -inf"
    g, r = gpu[vis], ref[vis]
    if r.size == 0:
        return
    bound = SCORE_REL * np.abs(r) + SCORE_FLOOR * np.abs(r).max()
    bad = np.abs(g - r) > bound
    say(f"  {what}: max rel err={float((np.abs(g - r) / np.maximum(np.abs(r), 1e-30)).max()):.3e}")
    assert not bad.any(), f"{what}: {int(bad.sum())} scores out of tolerance"


def assert_topk(gpu_idx: np.ndarray, ref_scores: np.ndarray, k: int, n_vis: int, what: str):
    """GPU selection (ascending, -1 padded) against float64 reference scores."""
    k_eff = min(k, n_vis)
    sel = gpu_idx[:k_eff]
    assert (gpu_idx[k_eff:] == -1).all(), f"{what}: padding"
    assert (np.diff(sel) > 0).all(), f"{what}: not strictly ascending"
    assert sel.min(initial=0) >= 0 and sel.max(initial=-1) < n_vis, f"{what}: index out of range"
    if k_eff == 0:
        return
    s = ref_scores[:n_vis]
    order = np.lexsort((np.arange(n_vis), -s))
    ref_set = set(order[:k_eff].tolist())
    sk = s[order[k_eff - 1]]
    diff = ref_set.symmetric_difference(sel.tolist())
    gap = max((abs(s[i] - sk) for i in diff), default=0.0)
    if diff:
        say(f"  {what}: {len(diff)} near-tie set differences, largest |s_i - s_k| = {gap:.2e}")
    far = [i for i in diff if abs(s[i] - sk) > TIE_ABS]
    assert not far, f"{what}: {len(far)} selection differences away from the k-th score (largest {gap:.3e})"
    return len(diff)
