"""Pins of the float64 merge (oracle/merge.py) to facts other than itself (CPU only).

The merge combines attention results of the same queries over disjoint key
chunks (the p2p ring step of TransformerEngine pull request 3527, section
Scope). What fixes it:

  split identity        merging per-chunk oracle results reproduces the
                        single-call oracle over all keys, for every mask,
                        GQA and packed batches (TL = TL chunk + BR chunk)
  neutral chunk         a chunk with LSE = -inf leaves the result unchanged
                        (pull request 3693, Description: neutral statistics
                        for empty ring blocks)
  all-empty rows        O = 0, LSE = -inf
  equal weights         two chunks with equal LSE: O = their mean,
                        LSE + ln 2
  order / grouping      permutations and nested merges agree
"""

import math

import numpy as np
import pytest
import torch

from oracle import MASK_CAUSAL_BR, MASK_CAUSAL_TL, MASK_NONE, lse_like_o, merge, sdpa_fwd
from oracle.floor import floor_merge


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def chunked(q, k, v, scale, bounds, masks, cu_q=None, cu_k=None):
    """Per-chunk oracle results for key ranges [bounds[i], bounds[i+1]) with the given masks.

    Dense only when cu_q is None; for packed inputs the key ranges are per sequence
    offsets (same split point inside every sequence)."""
    os_, ls = [], []
    for (lo, hi), m in zip(zip(bounds[:-1], bounds[1:]), masks):
        if cu_q is None:
            o, l = sdpa_fwd(q, k[:, lo:hi], v[:, lo:hi], m, scale)
        else:
            idx = np.concatenate([np.arange(cu_k[b] + lo, cu_k[b] + min(hi, cu_k[b + 1] - cu_k[b]))
                                  for b in range(len(cu_k) - 1)]).astype(np.int64)
            lens = [max(0, min(hi, cu_k[b + 1] - cu_k[b]) - lo) for b in range(len(cu_k) - 1)]
            ck = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
            o, l = sdpa_fwd(q, k[idx], v[idx], m, scale, cu_q, ck)
        os_.append(o)
        ls.append(lse_like_o(l, cu_q is not None))
    return os_, ls


@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2)])
def test_split_identity_no_mask(hq, hkv):
    q, k, v = rnd(1, 2, 7, hq, 8), rnd(2, 2, 11, hkv, 8), rnd(3, 2, 11, hkv, 8)
    o, l = sdpa_fwd(q, k, v, MASK_NONE, 0.3)
    os_, ls = chunked(q, k, v, 0.3, [0, 4, 5, 11], [MASK_NONE] * 3)
    mo, ml = merge(os_, ls)
    np.testing.assert_allclose(mo, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(ml, lse_like_o(l, False), rtol=0, atol=1e-13)


@pytest.mark.parametrize("split", [1, 5, 9])
def test_split_identity_causal_tl_is_tl_plus_br(split):
    # TL over S keys == TL over keys [0, c) merged with BR over keys [c, S): for query i the second
    # chunk's local key j' = j - c is allowed iff j' <= i + ((S - c) - S) = i - c.
    s = 12
    q, k, v = rnd(4, 1, s, 2, 4), rnd(5, 1, s, 2, 4), rnd(6, 1, s, 2, 4)
    o, l = sdpa_fwd(q, k, v, MASK_CAUSAL_TL, 0.5)
    os_, ls = chunked(q, k, v, 0.5, [0, split, s], [MASK_CAUSAL_TL, MASK_CAUSAL_BR])
    assert np.isneginf(ls[1][0, :split]).all()  # rows before the split see nothing in the second chunk
    mo, ml = merge(os_, ls)
    np.testing.assert_allclose(mo, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(ml, lse_like_o(l, False), rtol=0, atol=1e-13)


def test_split_identity_context_parallel_share():
    # BR over a long key range == full keys before the local block (no mask) + the local diagonal (TL)
    sq, skv = 6, 15
    q, k, v = rnd(7, 1, sq, 4, 8), rnd(8, 1, skv, 2, 8), rnd(9, 1, skv, 2, 8)
    o, l = sdpa_fwd(q, k, v, MASK_CAUSAL_BR, 0.4)
    os_, ls = chunked(q, k, v, 0.4, [0, skv - sq, skv], [MASK_NONE, MASK_CAUSAL_TL])
    mo, ml = merge(os_, ls)
    np.testing.assert_allclose(mo, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(ml, lse_like_o(l, False), rtol=0, atol=1e-13)


def test_split_identity_packed():
    lens = [5, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    t = int(cu[-1])
    q, k, v = rnd(10, t, 4, 8), rnd(11, t, 2, 8), rnd(12, t, 2, 8)
    o, l = sdpa_fwd(q, k, v, MASK_CAUSAL_TL, 0.35, cu, cu)
    # split every sequence's keys at 3: TL chunk [0, 3) and BR chunk [3, L) (empty for short sequences)
    os_, ls = chunked(q, k, v, 0.35, [0, 3, 10], [MASK_CAUSAL_TL, MASK_CAUSAL_BR], cu, cu)
    mo, ml = merge(os_, ls)
    np.testing.assert_allclose(mo, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(ml, l, rtol=0, atol=1e-13)


def test_neutral_chunk_and_single_chunk():
    o, l = rnd(13, 5, 3, 8), rnd(14, 5, 3)
    mo, ml = merge([o], [l])
    assert np.array_equal(ml, l) and np.allclose(mo, o, rtol=0, atol=1e-15)
    mo2, ml2 = merge([o, rnd(15, 5, 3, 8)], [l, np.full((5, 3), -np.inf)])
    assert np.array_equal(ml2, l) and np.array_equal(mo2, mo)


def test_all_empty_rows():
    mo, ml = merge([rnd(16, 4, 8), rnd(17, 4, 8)], [np.full(4, -np.inf), np.full(4, -np.inf)])
    assert np.isneginf(ml).all() and (mo == 0).all()


def test_equal_weights_closed_form():
    a, b = rnd(18, 3, 8), rnd(19, 3, 8)
    l = np.array([0.25, -3.0, 7.5])
    mo, ml = merge([a, b], [l, l])
    np.testing.assert_allclose(mo, (a + b) / 2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(ml, l + math.log(2.0), rtol=0, atol=1e-14)


def test_order_and_grouping():
    os_ = [rnd(20 + i, 6, 8) for i in range(3)]
    ls = [rnd(30 + i, 6) * 4 for i in range(3)]
    ls[1][2] = -np.inf
    m1 = merge(os_, ls)
    m2 = merge(os_[::-1], ls[::-1])
    ab = merge(os_[:2], ls[:2])
    m3 = merge([ab[0], os_[2]], [ab[1], ls[2]])
    for m in (m2, m3):
        np.testing.assert_allclose(m[0], m1[0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(m[1], m1[1], rtol=0, atol=1e-14)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_floor_merge_tracks_dtype(dtype):
    # the in-dtype merge differs from float64 by about the dtype's output rounding, and is not exact
    os_ = [torch.from_numpy(rnd(40 + i, 64, 16)).to(dtype) for i in range(3)]
    ls = [torch.from_numpy(rnd(50 + i, 64) * 3).to(torch.float32) for i in range(3)]
    fo, fl = floor_merge(os_, ls, dtype)
    ro, rl = merge([x.double().numpy() for x in os_], [x.double().numpy() for x in ls])
    err = np.abs(fo.double().numpy() - ro).max()
    ulp = 2.0 ** (-8 if dtype == torch.bfloat16 else -11)
    assert 0 < err <= ulp * max(1.0, np.abs(ro).max())
    assert np.abs(fl.double().numpy() - rl).max() < 1e-5
