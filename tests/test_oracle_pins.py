"""Pins of the float64 oracle to facts other than itself (CPU only).

Each test checks the oracle against something the mathematics or a hand
derivation fixes, chosen so that a plausible slip (a dropped term, a wrong
sign, a transposed operand, a log in the wrong base, a misplaced scale, a
diagonal on the wrong side) fails at least one of them:

  hand-worked example      tests/golden/hand_worked_d1.json (closed forms)
  finite differences       every gradient formula, scale placement, GQA sums
  V = identity             softmax rows sum to 1, P >= 0, masked P = 0
  K = 0 closed form        P = 1/n, O = prefix mean, LSE = ln n, dQ = 0, dV
  V = ones                 O = 1, dQ = dK = 0
  sum_j dK_j = 0           dS rows sum to zero
  K + 1 c^T shift          O unchanged, LSE shifts by scale q.c (natural log)
  TL == BR when Sq == Skv  alignment formulas
  context-parallel share   BR offset direction (all-gather rewrite)
  GQA == repeated-KV MHA   head mapping and dK/dV group sums
  packed == per-sequence   THD decomposition
  pair counts              closed-form allowed-pair counts
  floor                    in-dtype floor tracks the dtype's precision
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (MASK_CAUSAL_BR, MASK_CAUSAL_TL, MASK_NONE, allowed_pairs, count_allowed_pairs, head_backward,
                    head_forward, sdpa_bwd, sdpa_fwd)
from oracle.floor import floor_head, floor_units

HERE = os.path.dirname(os.path.abspath(__file__))
MASKS = {"none": MASK_NONE, "causal_tl": MASK_CAUSAL_TL, "causal_br": MASK_CAUSAL_BR}
ALL_MASKS = [MASK_NONE, MASK_CAUSAL_TL, MASK_CAUSAL_BR]


def rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- hand-worked

def _golden():
    with open(os.path.join(HERE, "golden", "hand_worked_d1.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden()["cases"], ids=lambda c: c["name"])
def test_hand_worked_example(case):
    scale = _golden()["common"]["scale"]
    m = MASKS[case["mask"]]
    q, k, v, do = (np.array(case[x], dtype=np.float64) for x in ("q", "k", "v", "do"))
    o, lse, _ = head_forward(q, k, v, scale, m)
    dq, dk, dv = head_backward(q, k, v, do, scale, m)
    exp_lse = np.array([float(x) for x in case["lse"]])
    np.testing.assert_allclose(o, case["o"], rtol=0, atol=1e-14)
    assert np.array_equal(np.isneginf(lse), np.isneginf(exp_lse))
    fin = np.isfinite(exp_lse)
    np.testing.assert_allclose(lse[fin], exp_lse[fin], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dq, case["dq"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dk, case["dk"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dv, case["dv"], rtol=0, atol=1e-14)


# ---------------------------------------------------------- finite differences

def _loss(q, k, v, do, mask, scale, cu_q=None, cu_k=None):
    o, _ = sdpa_fwd(q, k, v, mask, scale, cu_q, cu_k)
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


FD_CASES = [
    # (name, batch, hq, hkv, sq, skv, d, mask)
    ("none_sq", 1, 2, 2, 4, 4, 4, MASK_NONE),
    ("tl_sq", 1, 2, 2, 5, 5, 4, MASK_CAUSAL_TL),
    ("br_sq", 1, 2, 2, 5, 5, 8, MASK_CAUSAL_BR),
    ("tl_rect_q_lt_k", 2, 2, 1, 3, 6, 4, MASK_CAUSAL_TL),
    ("br_rect_q_lt_k", 1, 4, 2, 3, 6, 4, MASK_CAUSAL_BR),
    ("br_rect_q_gt_k_empty_rows", 1, 4, 2, 6, 3, 4, MASK_CAUSAL_BR),
    ("tl_rect_q_gt_k", 1, 2, 2, 6, 3, 8, MASK_CAUSAL_TL),
    ("none_gqa", 1, 4, 2, 4, 3, 4, MASK_NONE),
]


@pytest.mark.parametrize("case", FD_CASES, ids=lambda c: c[0])
def test_gradients_match_central_differences(case):
    _, b, hq, hkv, sq, skv, d, mask = case
    r = rng(11)
    q = r.standard_normal((b, sq, hq, d))
    k = r.standard_normal((b, skv, hkv, d))
    v = r.standard_normal((b, skv, hkv, d))
    do = r.standard_normal((b, sq, hq, d))
    scale = 0.7
    dq, dk, dv = sdpa_bwd(q, k, v, do, mask, scale)
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = _fd_grad(x, lambda: _loss(q, k, v, do, mask, scale))
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-7)


def test_gradients_match_central_differences_packed():
    r = rng(12)
    lens = [1, 3, 5]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    t = int(cu[-1])
    q = r.standard_normal((t, 4, 4))
    k = r.standard_normal((t, 2, 4))
    v = r.standard_normal((t, 2, 4))
    do = r.standard_normal((t, 4, 4))
    for mask in ALL_MASKS:
        dq, dk, dv = sdpa_bwd(q, k, v, do, mask, 0.5, cu, cu)
        for x, g in ((q, dq), (k, dk), (v, dv)):
            num = _fd_grad(x, lambda: _loss(q, k, v, do, mask, 0.5, cu, cu))
            np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-7)


# --------------------------------------------------------------- invariants

@pytest.mark.parametrize("mask", ALL_MASKS)
@pytest.mark.parametrize("shape", [(6, 6), (4, 9), (9, 4)])
def test_softmax_rows_via_identity_v(mask, shape):
    """With V = I (D = Skv), O is P itself: rows sum to 1, P >= 0, masked P = 0."""
    sq, skv = shape
    r = rng(13)
    q = r.standard_normal((sq, skv)) * 2
    k = r.standard_normal((skv, skv)) * 2
    o, lse, _ = head_forward(q, k, np.eye(skv), 0.9, mask)
    allow = allowed_pairs(sq, skv, mask)
    live = allow.any(axis=1)
    np.testing.assert_allclose(o[live].sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert (o >= 0).all()
    assert (o[~allow] == 0).all()
    assert (o[~live] == 0).all() and np.isneginf(lse[~live]).all()


@pytest.mark.parametrize("mask", ALL_MASKS)
@pytest.mark.parametrize("shape", [(7, 7), (5, 11), (11, 5)])
def test_zero_keys_closed_form(mask, shape):
    """K = 0: every allowed score is 0, so P = 1/n_i, O_i = mean of allowed v_j,
    LSE_i = ln n_i, dQ = 0, dV_j = sum over queries i that see j of dO_i / n_i."""
    sq, skv = shape
    r = rng(14)
    d = 3
    q = r.standard_normal((sq, d))
    k = np.zeros((skv, d))
    v = r.standard_normal((skv, d))
    do = r.standard_normal((sq, d))
    o, lse, _ = head_forward(q, k, v, 0.8, mask)
    dq, dk, dv = head_backward(q, k, v, do, 0.8, mask)
    for i in range(sq):
        if mask == MASK_NONE:
            hi = skv
        elif mask == MASK_CAUSAL_TL:
            hi = min(i + 1, skv)
        else:
            hi = max(0, min(i + skv - sq + 1, skv))
        if hi == 0:
            assert np.isneginf(lse[i]) and (o[i] == 0).all()
            continue
        np.testing.assert_allclose(o[i], v[:hi].mean(axis=0), rtol=0, atol=1e-12)
        assert abs(lse[i] - math.log(hi)) < 1e-12
    assert np.abs(dq).max() < 1e-12
    exp_dv = np.zeros((skv, d))
    for i in range(sq):
        n = int(allowed_pairs(sq, skv, mask)[i].sum())
        for j in range(skv):
            if allowed_pairs(sq, skv, mask)[i, j]:
                exp_dv[j] += do[i] / n
    np.testing.assert_allclose(dv, exp_dv, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mask", ALL_MASKS)
def test_constant_values(mask):
    """V = all ones: O = 1 on live rows, dQ = dK = 0 (dP is constant along j)."""
    r = rng(15)
    q = r.standard_normal((6, 5))
    k = r.standard_normal((8, 5))
    do = r.standard_normal((6, 5))
    o, lse, _ = head_forward(q, k, np.ones((8, 5)), 0.6, mask)
    dq, dk, _ = head_backward(q, k, np.ones((8, 5)), do, 0.6, mask)
    live = np.isfinite(lse)
    np.testing.assert_allclose(o[live], 1.0, rtol=0, atol=1e-12)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12


@pytest.mark.parametrize("mask", ALL_MASKS)
def test_dk_sums_to_zero(mask):
    """Each dS row sums to zero, so sum_j dK_j = scale * sum_i (sum_j dS_ij) q_i = 0."""
    r = rng(16)
    q = r.standard_normal((9, 6))
    k = r.standard_normal((12, 6))
    v = r.standard_normal((12, 6))
    do = r.standard_normal((9, 6))
    _, dk, _ = head_backward(q, k, v, do, 0.4, mask)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mask", ALL_MASKS)
def test_key_shift_invariance(mask):
    """K + 1 c^T adds scale * q_i.c to every score of row i: O is unchanged and
    the natural-log LSE_i moves by exactly scale * q_i.c (a log2 LSE would move by
    that times log2 e)."""
    r = rng(17)
    q = r.standard_normal((7, 4))
    k = r.standard_normal((10, 4))
    v = r.standard_normal((10, 4))
    c = r.standard_normal(4)
    scale = 0.55
    o1, l1, _ = head_forward(q, k, v, scale, mask)
    o2, l2, _ = head_forward(q, k + c[None, :], v, scale, mask)
    live = np.isfinite(l1)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2[live] - l1[live], scale * (q[live] @ c), rtol=0, atol=1e-12)


def test_tl_equals_br_when_square():
    r = rng(18)
    q, k, v, do = (r.standard_normal((1, 9, 2, 5)) for _ in range(4))
    a = sdpa_fwd(q, k, v, MASK_CAUSAL_TL, 0.3) + sdpa_bwd(q, k, v, do, MASK_CAUSAL_TL, 0.3)
    b = sdpa_fwd(q, k, v, MASK_CAUSAL_BR, 0.3) + sdpa_bwd(q, k, v, do, MASK_CAUSAL_BR, 0.3)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_tl_differs_from_br_when_rectangular():
    r = rng(19)
    q = r.standard_normal((1, 3, 1, 4))
    k, v = r.standard_normal((1, 7, 1, 4)), r.standard_normal((1, 7, 1, 4))
    o1, _ = sdpa_fwd(q, k, v, MASK_CAUSAL_TL, 0.5)
    o2, _ = sdpa_fwd(q, k, v, MASK_CAUSAL_BR, 0.5)
    assert np.abs(o1 - o2).max() > 1e-3


def test_context_parallel_share_identity():
    """All-gather context parallelism (pull request 3527, Approach): a rank holding
    the last Sq_loc queries against the full KV runs a bottom-right causal block.
    Its O/LSE/dQ equal the matching rows of top-left causal attention over the
    full sequence, and its dK/dV equal the full backward with dO zero elsewhere."""
    r = rng(20)
    s_full, s_loc, d = 16, 4, 5
    q_full = r.standard_normal((1, s_full, 2, d))
    k = r.standard_normal((1, s_full, 1, d))
    v = r.standard_normal((1, s_full, 1, d))
    do_full = np.zeros((1, s_full, 2, d))
    do_full[:, s_full - s_loc:] = r.standard_normal((1, s_loc, 2, d))
    q_loc, do_loc = q_full[:, s_full - s_loc:], do_full[:, s_full - s_loc:]
    o_l, lse_l = sdpa_fwd(q_loc, k, v, MASK_CAUSAL_BR, 0.45)
    o_f, lse_f = sdpa_fwd(q_full, k, v, MASK_CAUSAL_TL, 0.45)
    np.testing.assert_allclose(o_l, o_f[:, s_full - s_loc:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_l, lse_f[:, :, s_full - s_loc:], rtol=0, atol=1e-12)
    dq_l, dk_l, dv_l = sdpa_bwd(q_loc, k, v, do_loc, MASK_CAUSAL_BR, 0.45)
    dq_f, dk_f, dv_f = sdpa_bwd(q_full, k, v, do_full, MASK_CAUSAL_TL, 0.45)
    np.testing.assert_allclose(dq_l, dq_f[:, s_full - s_loc:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk_l, dk_f, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv_l, dv_f, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mask", ALL_MASKS)
def test_gqa_equals_repeated_kv_mha(mask):
    r = rng(21)
    hq, hkv = 6, 2
    q = r.standard_normal((2, 5, hq, 4))
    k = r.standard_normal((2, 7, hkv, 4))
    v = r.standard_normal((2, 7, hkv, 4))
    do = r.standard_normal((2, 5, hq, 4))
    kr, vr = np.repeat(k, hq // hkv, axis=2), np.repeat(v, hq // hkv, axis=2)
    o1, l1 = sdpa_fwd(q, k, v, mask, 0.5)
    o2, l2 = sdpa_fwd(q, kr, vr, mask, 0.5)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    dq1, dk1, dv1 = sdpa_bwd(q, k, v, do, mask, 0.5)
    dq2, dk2, dv2 = sdpa_bwd(q, kr, vr, do, mask, 0.5)
    np.testing.assert_allclose(dq1, dq2, rtol=0, atol=1e-13)
    g = hq // hkv
    np.testing.assert_allclose(dk1, dk2.reshape(2, 7, hkv, g, 4).sum(axis=3), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv1, dv2.reshape(2, 7, hkv, g, 4).sum(axis=3), rtol=0, atol=1e-12)


@pytest.mark.parametrize("mask", ALL_MASKS)
def test_packed_equals_per_sequence_dense(mask):
    r = rng(22)
    lq, lk = [3, 1, 6, 4], [5, 2, 6, 1]
    cq = np.concatenate([[0], np.cumsum(lq)])
    ck = np.concatenate([[0], np.cumsum(lk)])
    q = r.standard_normal((cq[-1], 4, 3))
    k = r.standard_normal((ck[-1], 2, 3))
    v = r.standard_normal((ck[-1], 2, 3))
    do = r.standard_normal((cq[-1], 4, 3))
    o, lse = sdpa_fwd(q, k, v, mask, 0.6, cq, ck)
    dq, dk, dv = sdpa_bwd(q, k, v, do, mask, 0.6, cq, ck)
    for b in range(4):
        qs, ks = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
        ob, lb = sdpa_fwd(q[None, qs], k[None, ks], v[None, ks], mask, 0.6)
        dqb, dkb, dvb = sdpa_bwd(q[None, qs], k[None, ks], v[None, ks], do[None, qs], mask, 0.6)
        np.testing.assert_array_equal(o[qs], ob[0])
        np.testing.assert_array_equal(lse[qs], lb[0].T)
        np.testing.assert_array_equal(dq[qs], dqb[0])
        np.testing.assert_allclose(dk[ks], dkb[0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(dv[ks], dvb[0], rtol=0, atol=1e-13)


def test_unit_sampling_matches_full():
    r = rng(23)
    q = r.standard_normal((2, 6, 4, 3))
    k = r.standard_normal((2, 6, 2, 3))
    v = r.standard_normal((2, 6, 2, 3))
    do = r.standard_normal((2, 6, 4, 3))
    o, lse = sdpa_fwd(q, k, v, MASK_CAUSAL_TL, 0.5)
    dq, dk, dv = sdpa_bwd(q, k, v, do, MASK_CAUSAL_TL, 0.5)
    os_, ls_ = sdpa_fwd(q, k, v, MASK_CAUSAL_TL, 0.5, units=[(1, 0)])
    dqs, dks, dvs = sdpa_bwd(q, k, v, do, MASK_CAUSAL_TL, 0.5, units=[(1, 0)])
    np.testing.assert_array_equal(os_[1, :, 0:2], o[1, :, 0:2])
    np.testing.assert_array_equal(ls_[1, 0:2], lse[1, 0:2])
    np.testing.assert_array_equal(dks[1, :, 0], dk[1, :, 0])
    np.testing.assert_array_equal(dqs[1, :, 0:2], dq[1, :, 0:2])
    assert np.isnan(os_[0]).all() and np.isnan(dvs[1, :, 1]).all()


# ------------------------------------------------------------- pair counts

def test_pair_counts_brute_force():
    for sq, skv in [(1, 1), (5, 5), (3, 8), (8, 3), (17, 33)]:
        for m in ALL_MASKS:
            assert count_allowed_pairs([sq], [skv], m) == int(allowed_pairs(sq, skv, m).sum())


def test_pair_counts_closed_forms_at_workload_sizes():
    # causal top-left square: S(S+1)/2 per head
    assert count_allowed_pairs([8192], [8192], MASK_CAUSAL_TL) == 8192 * 8193 // 2
    assert 2 * 16 * count_allowed_pairs([8192], [8192], MASK_CAUSAL_TL) == 1_073_872_896
    # bottom-right Sq=4096 vs Skv=16384: row i sees i + 12289 keys
    assert count_allowed_pairs([4096], [16384], MASK_CAUSAL_BR) == 4096 * 12289 + 4095 * 4096 // 2
    assert count_allowed_pairs([4096], [16384], MASK_CAUSAL_TL) == 4096 * 4097 // 2


# ------------------------------------------------------------------- floor

@pytest.mark.parametrize("dtype,eps", [(torch.bfloat16, 2.0 ** -8), (torch.float16, 2.0 ** -11)])
def test_floor_tracks_dtype_precision(dtype, eps):
    """The floor's error against float64 is a few ulps of the dtype: nonzero (it
    really rounds) and small (it computes the same function)."""
    g = torch.Generator().manual_seed(5)
    sq, skv, d = 48, 64, 32
    q, k, v, do = (torch.randn(s, d, generator=g).to(dtype) for s in (sq, skv, skv, sq))
    scale = d ** -0.5
    o, lse, dq, dk, dv = floor_head(q, k, v, do, scale, MASK_CAUSAL_BR, dtype)
    f64 = [x.double().numpy() for x in (q, k, v, do)]
    ro, rl, _ = head_forward(*f64[:3], scale, MASK_CAUSAL_BR)
    rdq, rdk, rdv = head_backward(*f64, scale, MASK_CAUSAL_BR)
    for got, ref in ((o, ro), (dq, rdq), (dk, rdk), (dv, rdv)):
        err = np.abs(got.double().numpy() - ref).max()
        mag = np.abs(ref).max()
        assert 0 < err < 40 * eps * mag
    assert np.abs(lse.double().numpy() - rl).max() < 40 * eps * np.abs(rl).max()


def test_floor_in_fp32_is_the_oracle():
    g = torch.Generator().manual_seed(6)
    q, k, v, do = (torch.randn(s, 16, generator=g) for s in (20, 30, 30, 20))
    o, lse, dq, dk, dv = floor_head(q, k, v, do, 0.25, MASK_CAUSAL_TL, torch.float32)
    f64 = [x.double().numpy() for x in (q, k, v, do)]
    ro, rl, _ = head_forward(*f64[:3], 0.25, MASK_CAUSAL_TL)
    rdq, rdk, rdv = head_backward(*f64, 0.25, MASK_CAUSAL_TL)
    for got, ref in ((o, ro), (lse, rl), (dq, rdq), (dk, rdk), (dv, rdv)):
        np.testing.assert_allclose(got.double().numpy(), ref, rtol=1e-4, atol=1e-5)


def test_floor_units_group_sums():
    g = torch.Generator().manual_seed(7)
    q = torch.randn(1, 10, 4, 8, generator=g)
    k = torch.randn(1, 12, 2, 8, generator=g)
    v = torch.randn(1, 12, 2, 8, generator=g)
    do = torch.randn(1, 10, 4, 8, generator=g)
    res = floor_units(q, k, v, do, MASK_CAUSAL_BR, 0.3, torch.float32, [(0, 1)])
    _, rdk, rdv = sdpa_bwd(q.double().numpy(), k.double().numpy(), v.double().numpy(), do.double().numpy(),
                           MASK_CAUSAL_BR, 0.3, units=[(0, 1)])
    np.testing.assert_allclose(res[(0, 1)]["dk"].double().numpy(), rdk[0, :, 1], rtol=1e-4, atol=1e-5)
    np.testing.assert_allclose(res[(0, 1)]["dv"].double().numpy(), rdv[0, :, 1], rtol=1e-4, atol=1e-5)
