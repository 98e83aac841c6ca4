"""Pins of the head-dim reading of the float64 oracle (CPU only).

TransformerEngine pull request 3527, section Scope: the backward engine there
serves any head dim that is a multiple of 8 up to 512 by padding to its
compiled width, is held to d_qk == d_v only by an engine flag, and the forward
engine lists the asymmetric pair (192, 128). Reading: Q and K share D_qk, V and
O (so dO and dV) have their own D_v, and nothing but the dot products depends
on either. What fixes it here, independently of the oracle's own code:

  V-column split     attention with V = [V1 | V2] is [O1 | O2] with the same
                     LSE; with dO = [dO1 | dO2] the gradients are dQ1 + dQ2,
                     dK1 + dK2 and [dV1 | dV2] (dP and its row sum D are sums
                     over V's columns)
  zero padding       Q, K padded with zero columns and V, dO with zero columns
                     give the unpadded results on the real columns and exact
                     zeros on the padded ones (how a kernel built for a wider
                     head computes a narrower one)
  K = 0              O_i = mean of the allowed v_j at any D_v, LSE = ln n_i,
                     dQ = 0, dV_j = sum of dO_i / n_i
  gradients          central finite differences with D_qk != D_v (every mask,
                     GQA, rectangular, window, packed)
  declines           Q/K head dims that differ; K/V or dO shapes that do not fit
"""

import numpy as np
import pytest

from oracle import MASK_CAUSAL_BR, MASK_CAUSAL_TL, MASK_NONE, allowed_pairs, head_backward, head_forward, sdpa_bwd, sdpa_fwd

MASKS = [MASK_NONE, MASK_CAUSAL_TL, MASK_CAUSAL_BR]


def rng(seed):
    return np.random.default_rng(seed)


@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("shape", [(7, 7), (5, 9), (9, 4)])
def test_v_column_split(mask, shape):
    sq, skv = shape
    r = rng(11)
    b, hq, hkv, dqk, d1, d2 = 2, 4, 2, 6, 3, 5
    q, k = r.standard_normal((b, sq, hq, dqk)), r.standard_normal((b, skv, hkv, dqk))
    v1, v2 = r.standard_normal((b, skv, hkv, d1)), r.standard_normal((b, skv, hkv, d2))
    do1, do2 = r.standard_normal((b, sq, hq, d1)), r.standard_normal((b, sq, hq, d2))
    v, do = np.concatenate([v1, v2], axis=-1), np.concatenate([do1, do2], axis=-1)
    o, lse = sdpa_fwd(q, k, v, mask, 0.45)
    o1, lse1 = sdpa_fwd(q, k, v1, mask, 0.45)
    o2, lse2 = sdpa_fwd(q, k, v2, mask, 0.45)
    np.testing.assert_array_equal(lse, lse1)
    np.testing.assert_array_equal(lse, lse2)
    np.testing.assert_allclose(o, np.concatenate([o1, o2], axis=-1), rtol=0, atol=1e-14)
    dq, dk, dv = sdpa_bwd(q, k, v, do, mask, 0.45)
    dq1, dk1, dv1 = sdpa_bwd(q, k, v1, do1, mask, 0.45)
    dq2, dk2, dv2 = sdpa_bwd(q, k, v2, do2, mask, 0.45)
    np.testing.assert_allclose(dq, dq1 + dq2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk, dk1 + dk2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv, np.concatenate([dv1, dv2], axis=-1), rtol=0, atol=1e-14)


@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("dims", [(8, 8, 64, 64), (24, 16, 32, 32), (6, 10, 16, 64)])
def test_zero_padding_keeps_the_real_columns(mask, dims):
    dqk, dv, pqk, pv = dims
    r = rng(12)
    sq, skv = 6, 8
    q, k = r.standard_normal((sq, dqk)), r.standard_normal((skv, dqk))
    v, do = r.standard_normal((skv, dv)), r.standard_normal((sq, dv))

    def pad(x, width):
        return np.concatenate([x, np.zeros((x.shape[0], width - x.shape[1]))], axis=1)

    o, lse, _ = head_forward(q, k, v, 0.3, mask)
    po, plse, _ = head_forward(pad(q, pqk), pad(k, pqk), pad(v, pv), 0.3, mask)
    np.testing.assert_allclose(po[:, :dv], o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(plse, lse, rtol=0, atol=1e-14)
    assert (po[:, dv:] == 0).all()
    dq, dk, dvv = head_backward(q, k, v, do, 0.3, mask)
    pdq, pdk, pdv = head_backward(pad(q, pqk), pad(k, pqk), pad(v, pv), pad(do, pv), 0.3, mask)
    for full, real, width in ((pdq, dq, dqk), (pdk, dk, dqk), (pdv, dvv, dv)):
        np.testing.assert_allclose(full[:, :width], real, rtol=0, atol=1e-13)
        assert (full[:, width:] == 0).all()


@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("dims", [(3, 7), (8, 2)])
def test_zero_keys_closed_form_asymmetric(mask, dims):
    dqk, dv = dims
    r = rng(13)
    sq, skv = 5, 9
    q, v, do = r.standard_normal((sq, dqk)), r.standard_normal((skv, dv)), r.standard_normal((sq, dv))
    k = np.zeros((skv, dqk))
    allow = allowed_pairs(sq, skv, mask)
    o, lse, _ = head_forward(q, k, v, 0.8, mask)
    dq, dk, dvv = head_backward(q, k, v, do, 0.8, mask)
    exp_dv = np.zeros((skv, dv))
    for i in range(sq):
        keys = [j for j in range(skv) if allow[i, j]]
        np.testing.assert_allclose(o[i], v[keys].mean(axis=0), rtol=0, atol=1e-12)
        assert abs(lse[i] - np.log(len(keys))) < 1e-12
        for j in keys:
            exp_dv[j] += do[i] / len(keys)
    assert o.shape == (sq, dv) and dq.shape == (sq, dqk) and dk.shape == (skv, dqk)
    assert np.abs(dq).max() < 1e-12
    np.testing.assert_allclose(dvv, exp_dv, rtol=0, atol=1e-12)


def _loss(q, k, v, do, mask, scale, w=-1, cu=None):
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
    ("none", MASK_NONE, 1, 2, 2, 4, 5, 6, 3, -1),
    ("tl_gqa", MASK_CAUSAL_TL, 2, 4, 2, 5, 5, 2, 5, -1),
    ("br_rect", MASK_CAUSAL_BR, 1, 2, 1, 3, 6, 5, 3, -1),
    ("br_empty_rows", MASK_CAUSAL_BR, 1, 2, 2, 6, 3, 3, 4, -1),
    ("tl_window", MASK_CAUSAL_TL, 1, 2, 1, 6, 6, 4, 2, 1),
], ids=lambda c: c[0])
def test_gradients_match_central_differences_asymmetric(case):
    _, mask, b, hq, hkv, sq, skv, dqk, dv, w = case
    r = rng(14)
    q, k = r.standard_normal((b, sq, hq, dqk)), r.standard_normal((b, skv, hkv, dqk))
    v, do = r.standard_normal((b, skv, hkv, dv)), r.standard_normal((b, sq, hq, dv))
    dq, dk, dvv = sdpa_bwd(q, k, v, do, mask, 0.6, window_left=w)
    for x, g in ((q, dq), (k, dk), (v, dvv)):
        num = _fd_grad(x, lambda: _loss(q, k, v, do, mask, 0.6, w))
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-7)


def test_gradients_match_central_differences_packed_asymmetric():
    r = rng(15)
    lens = [2, 5]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    t = int(cu[-1])
    q, k = r.standard_normal((t, 2, 3)), r.standard_normal((t, 1, 3))
    v, do = r.standard_normal((t, 1, 5)), r.standard_normal((t, 2, 5))
    for mask in (MASK_CAUSAL_TL, MASK_CAUSAL_BR):
        dq, dk, dv = sdpa_bwd(q, k, v, do, mask, 0.5, cu, cu)
        for x, g in ((q, dq), (k, dk), (v, dv)):
            num = _fd_grad(x, lambda: _loss(q, k, v, do, mask, 0.5, -1, cu))
            np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-7)


def test_shape_declines():
    r = rng(16)
    q, k = r.standard_normal((1, 4, 2, 8)), r.standard_normal((1, 4, 2, 8))
    with pytest.raises(ValueError):  # Q and K must share D_qk
        sdpa_fwd(q, r.standard_normal((1, 4, 2, 6)), r.standard_normal((1, 4, 2, 8)), MASK_NONE, 0.5)
    with pytest.raises(ValueError):  # V must match K's tokens and heads
        sdpa_fwd(q, k, r.standard_normal((1, 5, 2, 8)), MASK_NONE, 0.5)
    with pytest.raises(ValueError):  # dO has O's shape: Q's layout with V's head dim
        sdpa_bwd(q, k, r.standard_normal((1, 4, 2, 4)), r.standard_normal((1, 4, 2, 8)), MASK_NONE, 0.5)
