"""Pins of the sliding-window reading of the float64 oracle (CPU only).

TransformerEngine pull request 3527, section Scope: sliding windows are
supported with the all-gather and a2a context-parallel modes, measured against
the top-left or bottom-right diagonal (Known limitations). Reading: a causal
mask with window W >= 0 admits key j for query i iff
i + delta - W <= j <= i + delta (delta = 0 TL, Skv - Sq BR). What fixes it
here, independently of the oracle's own code:

  wide window      W >= Skv + |delta| reproduces the plain causal mask exactly
  W = 0            every live row sees only its diagonal key: O_i = v_{i+delta},
                   LSE_i = S_{i,i+delta}, empty rows where i + delta is outside
  K = 0            P = 1/n_i over the window, O_i = window mean, LSE = ln n_i,
                   dV_j = sum over the rows whose window holds j of dO_i / n_i,
                   with n_i counted by hand from the definition
  gradients        central finite differences (TL, BR, GQA, rectangular,
                   packed) with windows
  pair counts      closed form against brute force
  declines         a window without a causal mask
"""

import math

import numpy as np
import pytest

from oracle import (MASK_CAUSAL_BR, MASK_CAUSAL_TL, MASK_NONE, allowed_pairs, count_allowed_pairs, head_backward,
                    head_forward, sdpa_bwd, sdpa_fwd)

CAUSAL = [MASK_CAUSAL_TL, MASK_CAUSAL_BR]
SHAPES = [(9, 9), (5, 12), (12, 5)]


def rng(seed):
    return np.random.default_rng(seed)


def _delta(mask, sq, skv):
    return 0 if mask == MASK_CAUSAL_TL else skv - sq


def _window_by_hand(i, mask, sq, skv, w):
    """The keys of row i, listed from the reading (not from allowed_pairs)."""
    dlt = _delta(mask, sq, skv)
    return [j for j in range(skv) if i + dlt - w <= j <= i + dlt]


@pytest.mark.parametrize("mask", CAUSAL)
@pytest.mark.parametrize("shape", SHAPES)
def test_wide_window_is_the_causal_mask(mask, shape):
    sq, skv = shape
    r = rng(1)
    q, k, v = r.standard_normal((sq, 4)), r.standard_normal((skv, 4)), r.standard_normal((skv, 4))
    w = skv + abs(skv - sq)
    assert np.array_equal(allowed_pairs(sq, skv, mask, w), allowed_pairs(sq, skv, mask))
    o1, l1, _ = head_forward(q, k, v, 0.6, mask, w)
    o2, l2, _ = head_forward(q, k, v, 0.6, mask)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("mask", CAUSAL)
@pytest.mark.parametrize("shape", SHAPES)
def test_zero_window_sees_only_the_diagonal(mask, shape):
    sq, skv = shape
    r = rng(2)
    q, k, v = r.standard_normal((sq, 4)), r.standard_normal((skv, 4)), r.standard_normal((skv, 4))
    o, lse, _ = head_forward(q, k, v, 0.9, mask, 0)
    dlt = _delta(mask, sq, skv)
    for i in range(sq):
        j = i + dlt
        if 0 <= j < skv:
            np.testing.assert_allclose(o[i], v[j], rtol=0, atol=1e-14)
            assert abs(lse[i] - 0.9 * float(q[i] @ k[j])) < 1e-13
        else:
            assert np.isneginf(lse[i]) and (o[i] == 0).all()


@pytest.mark.parametrize("mask", CAUSAL)
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("w", [1, 3])
def test_zero_keys_closed_form_with_window(mask, shape, w):
    sq, skv = shape
    r = rng(3)
    d = 3
    q, v, do = r.standard_normal((sq, d)), r.standard_normal((skv, d)), r.standard_normal((sq, d))
    k = np.zeros((skv, d))
    o, lse, _ = head_forward(q, k, v, 0.8, mask, w)
    dq, _, dv = head_backward(q, k, v, do, 0.8, mask, w)
    exp_dv = np.zeros((skv, d))
    for i in range(sq):
        keys = _window_by_hand(i, mask, sq, skv, w)
        if not keys:
            assert np.isneginf(lse[i]) and (o[i] == 0).all()
            continue
        np.testing.assert_allclose(o[i], v[keys].mean(axis=0), rtol=0, atol=1e-12)
        assert abs(lse[i] - math.log(len(keys))) < 1e-12
        for j in keys:
            exp_dv[j] += do[i] / len(keys)
    assert np.abs(dq).max() < 1e-12
    np.testing.assert_allclose(dv, exp_dv, rtol=0, atol=1e-12)


def _loss(q, k, v, do, mask, scale, w, cu=None):
    o, _ = sdpa_fwd(q, k, v, mask, scale, cu, cu, window_left=w)
    return float(np.nansum(o * do))


def _fd_grad(x, f, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        old = x[idx]
        x[idx] = old + h
        fp = f()
        x[idx] = old - h
        fm = f()
        x[idx] = old
        g[idx] = (fp - fm) / (2 * h)
    return g


@pytest.mark.parametrize("case", [
    ("tl", MASK_CAUSAL_TL, 1, 2, 2, 6, 6, 2),
    ("br_rect", MASK_CAUSAL_BR, 1, 4, 2, 4, 7, 1),
    ("tl_rect_gqa", MASK_CAUSAL_TL, 2, 4, 2, 6, 4, 2),
    ("br_empty_rows", MASK_CAUSAL_BR, 1, 2, 1, 6, 3, 1),
], ids=lambda c: c[0])
def test_gradients_match_central_differences_with_window(case):
    _, mask, b, hq, hkv, sq, skv, w = case
    r = rng(4)
    q, k = r.standard_normal((b, sq, hq, 4)), r.standard_normal((b, skv, hkv, 4))
    v, do = r.standard_normal((b, skv, hkv, 4)), r.standard_normal((b, sq, hq, 4))
    dq, dk, dv = sdpa_bwd(q, k, v, do, mask, 0.7, window_left=w)
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = _fd_grad(x, lambda: _loss(q, k, v, do, mask, 0.7, w))
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-7)


def test_gradients_match_central_differences_packed_window():
    r = rng(5)
    lens = [1, 4, 6]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    t = int(cu[-1])
    q, k = r.standard_normal((t, 2, 4)), r.standard_normal((t, 1, 4))
    v, do = r.standard_normal((t, 1, 4)), r.standard_normal((t, 2, 4))
    for mask in CAUSAL:
        dq, dk, dv = sdpa_bwd(q, k, v, do, mask, 0.5, cu, cu, window_left=2)
        for x, g in ((q, dq), (k, dk), (v, dv)):
            num = _fd_grad(x, lambda: _loss(q, k, v, do, mask, 0.5, 2, cu))
            np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("mask", CAUSAL)
def test_pair_counts_with_window(mask):
    for sq, skv in [(9, 9), (5, 12), (12, 5), (1, 7), (7, 1)]:
        for w in [0, 1, 2, 5, 50]:
            brute = int(allowed_pairs(sq, skv, mask, w).sum())
            hand = sum(len(_window_by_hand(i, mask, sq, skv, w)) for i in range(sq))
            assert brute == hand == count_allowed_pairs([sq], [skv], mask, w)


def test_window_needs_a_causal_mask():
    with pytest.raises(ValueError):
        allowed_pairs(4, 4, MASK_NONE, 2)
    with pytest.raises(ValueError):
        count_allowed_pairs([4], [4], MASK_NONE, 2)
