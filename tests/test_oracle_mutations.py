"""Mutation checks: plant a plausible mistake in the oracle (on the CPU) and show a pin catches it."""
import numpy as np
import pytest

from oracle import attention as oa
from oracle import compress as oc
from oracle import indexer as oi

import test_oracle_attention as ta
import test_oracle_compress as tc
import test_oracle_indexer as ti


def _rope_half_split(x, pos, rope_dim, base=10000.0):
    x = np.array(x, dtype=np.float64, copy=True)
    D = x.shape[-1]
    h = rope_dim // 2
    theta = base ** (-2.0 * np.arange(h) / rope_dim)
    phi = np.asarray(pos, dtype=np.float64)[..., None] * theta
    a = x[..., D - rope_dim:D - h].copy()
    b = x[..., D - h:].copy()
    x[..., D - rope_dim:D - h] = a * np.cos(phi) - b * np.sin(phi)
    x[..., D - h:] = a * np.sin(phi) + b * np.cos(phi)
    return x


def _rope_wrong_freq(x, pos, rope_dim, base=10000.0):
    return _ORIG_ROPE(x, pos, rope_dim, base ** 0.5)


_ORIG_ROPE = oc.rope


@pytest.mark.parametrize("bad", [_rope_half_split, _rope_wrong_freq])
def test_rope_mutations_fail_the_gptj_pin(monkeypatch, bad):
    monkeypatch.setattr(oc, "rope", bad)
    with pytest.raises(AssertionError):
        tc.test_rope_matches_gptj_interleaved_rotary(16, 64)


def test_dropped_overlap_fails_the_slot_pin(monkeypatch):
    orig = oc.entry_tokens
    monkeypatch.setattr(oc, "entry_tokens", lambda i, m, overlap: orig(i, m, 0))
    with pytest.raises(Exception):
        tc.test_bias_slot_layout_with_overlap(1)


def test_reversed_slots_fail_the_slot_pin(monkeypatch):
    orig = oc.entry_tokens

    def rev(i, m, overlap):
        toks, slots = orig(i, m, overlap)
        n = (1 + overlap) * m
        return toks, [n - 1 - s for s in slots]
    monkeypatch.setattr(oc, "entry_tokens", rev)
    with pytest.raises(AssertionError):
        tc.test_bias_slot_layout_with_overlap(6)


def test_entry_position_shift_fails_the_rotation_pin(monkeypatch):
    orig = oc.rope
    monkeypatch.setattr(oc, "compress", lambda c, z, bias, m, overlap, rope_dim, *a, **k: (
        _shifted_compress(orig, c, z, bias, m, overlap, rope_dim, *a, **k)))
    with pytest.raises(AssertionError):
        tc.test_compress_places_entries_at_their_group_start_and_chunks_agree()


def _shifted_compress(rope, c, z, bias, m, overlap, rope_dim, norm_w=None, eps=1e-6, rope_base=10000.0,
                      pos_first=0):
    lo, hi = oc.entry_range(pos_first, c.shape[0], m, overlap)
    pooled = np.stack([oc.pool_entry(c, z, bias, i, m, overlap, pos_first)[0] for i in range(lo, hi)])
    pos = (np.arange(lo, hi) + 1) * m - 1          # mistake: last token of the group
    return rope(oc.rms_norm(pooled, norm_w, eps), pos, rope_dim, rope_base), lo, pooled


def test_dropped_relu_fails_the_identity_pin(monkeypatch):
    def no_relu(q, w, k, n):
        s = np.full(k.shape[0], -np.inf)
        s[:n] = (k[:n] @ q.T) @ w
        return s
    monkeypatch.setattr(oi, "index_scores", no_relu)
    with pytest.raises(AssertionError):
        ti.test_relu_identities_pin_sign_and_weighting()


def test_weight_inside_relu_fails_the_identity_pin(monkeypatch):
    def w_inside(q, w, k, n):
        s = np.full(k.shape[0], -np.inf)
        s[:n] = np.maximum((k[:n] @ q.T) * w, 0).sum(1)
        return s
    monkeypatch.setattr(oi, "index_scores", w_inside)
    with pytest.raises(AssertionError):
        ti.test_relu_identities_pin_sign_and_weighting()


def test_dropped_window_fails_the_dense_reduction(monkeypatch):
    orig = oa.gather_rows

    def no_window(entries, sel, win_rows, win_pos0, t, window):
        X = orig(entries, sel, win_rows, win_pos0, t, window)
        n_sel = len([i for i in sel if i >= 0])
        return X[:max(n_sel, 1)]
    monkeypatch.setattr(oa, "gather_rows", no_window)
    with pytest.raises(AssertionError):
        ta.test_full_selection_and_full_window_reduce_to_dense_attention()


def test_unnormalised_query_fails_the_dense_reduction(monkeypatch):
    monkeypatch.setattr(oa, "prepare_query", lambda q, t, r, *a, **k: oc.rope(q, t, r))
    with pytest.raises(AssertionError):
        ta.test_full_selection_and_full_window_reduce_to_dense_attention()
