"""GPU parity of attn_merge: combining forward results over disjoint key chunks.

The p2p (ring) context-parallel mode of TransformerEngine pull request 3527
(section Scope) shards the keys across steps; every step is an attention call
over one key chunk and the steps' (O, LSE) are combined (oracle/merge.py), with
empty chunks neutral (pull request 3693, Description). Cases:

  * attn_merge alone on random parts (some rows empty in every part, one part
    half empty), dense and packed, D in {64, 128, 256, 512}, bf16 / fp16,
    1..8 parts, against the float64 merge; in place equals out of place;
  * split identity end to end: attn_fwd on two key chunks + attn_merge equals
    attention over all keys (no mask; TL = TL chunk + BR chunk; the
    context-parallel BR share = full chunk + TL chunk; a packed batch);
  * ring backward: attn_bwd per chunk with the merged O and LSE gives dK, dV
    of the chunk and a partial dQ whose sum is the full dQ.

Acceptance as in parity_util.compare. The floor of a merged result is the
in-dtype floor of each chunk merged by floor_merge (the parts are rounded to
the dtype before the merge, as on the GPU). Reading for the ring backward: dQ
is the sum of per-chunk dQ that were each rounded to the dtype, one rounding
more than the single call, so its error is held to 3x the single-call floor.
"""

import numpy as np
import pytest
import torch

import scaled_dot_product_02_amd as sd
from oracle import MASK_CAUSAL_BR, MASK_CAUSAL_TL, MASK_NONE, lse_like_o, merge, sdpa_bwd, sdpa_fwd
from oracle.floor import floor_head, floor_merge

from parity_util import BOUND, compare, f64

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "fp16": torch.float16}
DEV = torch.device("cuda:0")


def _rand_parts(n, o_shape, l_shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    os_ = [torch.randn(o_shape, generator=g).to(dtype) for _ in range(n)]
    ls = [(torch.randn(l_shape, generator=g) * 4).float() for _ in range(n)]
    for x in ls:  # a few rows are empty in every part
        x.view(-1)[::17] = float("-inf")
    if n > 1:  # one part is empty on half of the rows
        ls[1].view(-1)[::2] = float("-inf")
    return os_, ls


def _check(name, got_o, got_l, ref_o, ref_l, flo_o, flo_l, dtype):
    ok1, m1 = compare(f"{name} O", got_o, ref_o, flo_o, dtype)
    ok2, m2 = compare(f"{name} LSE", got_l, ref_l, flo_l, dtype, is_lse=True)
    print("   ", m1)
    print("   ", m2)
    assert ok1 and ok2, (m1, m2)


@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("n", [1, 2, 3, 8])
@pytest.mark.parametrize("packed", [False, True])
def test_merge_random_parts(d, dtype, n, packed):
    if packed:
        lens = [40, 1, 77]
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
        o_shape, l_shape = (sum(lens), 3, d), (sum(lens), 3)
    else:
        cu = None
        o_shape, l_shape = (2, 61, 3, d), (2, 3, 61)
    os_, ls = _rand_parts(n, o_shape, l_shape, DT[dtype], seed=d + 7 * n + (100 if packed else 0))
    go, gl = sd.attn_merge([x.to(DEV) for x in os_], [x.to(DEV) for x in ls],
                           cu_seqlens_q=None if cu is None else cu.to(DEV))
    torch.cuda.synchronize()
    ref_o, ref_l = merge([f64(x) for x in os_], [lse_like_o(f64(x), packed) for x in ls])
    fo, fl = floor_merge(os_, [torch.from_numpy(lse_like_o(x.numpy(), packed)) for x in ls], DT[dtype])
    _check(f"merge d{d} {dtype} n{n}", f64(go), lse_like_o(f64(gl), packed), ref_o, ref_l,
           fo.double().numpy(), fl.double().numpy(), dtype)


def test_merge_in_place_equals_out_of_place():
    os_, ls = _rand_parts(3, (2, 50, 4, 128), (2, 4, 50), torch.bfloat16, seed=5)
    po = [x.to(DEV) for x in os_]
    pl = [x.to(DEV) for x in ls]
    ro, rl = sd.attn_merge(po, pl)
    io, il = sd.attn_merge(po, pl, out=po[0], lse=pl[0])
    torch.cuda.synchronize()
    assert io.data_ptr() == po[0].data_ptr() and il.data_ptr() == pl[0].data_ptr()
    assert torch.equal(io.cpu(), ro.cpu())
    assert torch.equal(torch.nan_to_num(il.cpu(), neginf=-1e30), torch.nan_to_num(rl.cpu(), neginf=-1e30))


def test_merge_declines_partial_overlap():
    os_, ls = _rand_parts(2, (1, 32, 2, 64), (1, 2, 32), torch.bfloat16, seed=6)
    n = os_[0].numel()
    buf = torch.empty(2 * n, dtype=torch.bfloat16, device=DEV)
    po = [buf[:n].view(os_[0].shape), os_[1].to(DEV)]
    po[0].copy_(os_[0].to(DEV))
    pl = [x.to(DEV) for x in ls]
    shifted = buf[n // 2:n // 2 + n].view(os_[0].shape)  # same layout, half inside part 0
    with pytest.raises(sd.AttnError) as e:
        sd.attn_merge(po, pl, out=shifted)
    assert e.value.status_name == "ATTN_E_OVERLAP"


def _floor_chunk(q, k, v, mask, scale, dtype):
    """In-dtype floor of one forward call, dense [B,S,H,D] inputs: returns O [B,Sq,Hq,D], LSE [B,Sq,Hq]."""
    b, sq, hq, d = q.shape
    hkv = k.shape[2]
    grp = hq // hkv
    o = torch.zeros(b, sq, hq, d)
    lse = torch.zeros(b, sq, hq)
    dummy = torch.zeros(sq, d, dtype=dtype)
    for bi in range(b):
        for h in range(hq):
            fo, fl, *_ = floor_head(q[bi, :, h], k[bi, :, h // grp], v[bi, :, h // grp], dummy, scale, mask, dtype)
            o[bi, :, h] = fo
            lse[bi, :, h] = fl
    return o.to(dtype), lse


SPLITS = [
    # (mask of the full call, sq, skv, split, mask of chunk 1, mask of chunk 2)
    ("none", 200, 333, 150, "none", "none"),
    ("causal_tl", 333, 333, 100, "causal_tl", "causal_br"),
    ("causal_br", 200, 333, 133, "none", "causal_tl"),
]
MASK = {"none": MASK_NONE, "causal_tl": MASK_CAUSAL_TL, "causal_br": MASK_CAUSAL_BR}


def _inputs(sq, skv, hq, hkv, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(2, sq, hq, d, generator=g).to(DT[dtype])
    k = torch.randn(2, skv, hkv, d, generator=g).to(DT[dtype])
    v = torch.randn(2, skv, hkv, d, generator=g).to(DT[dtype])
    do = torch.randn(2, sq, hq, d, generator=g).to(DT[dtype])
    return q, k, v, do


@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("split", SPLITS, ids=lambda s: s[0])
def test_split_identity_forward(d, dtype, split):
    full, sq, skv, c, m1, m2 = split
    q, k, v, _ = _inputs(sq, skv, 4, 2, d, dtype, seed=d + sq)
    scale = d ** -0.5
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o1, l1 = sd.attn_fwd(qd, kd[:, :c].contiguous(), vd[:, :c].contiguous(), mask=m1, scale=scale)
    o2, l2 = sd.attn_fwd(qd, kd[:, c:].contiguous(), vd[:, c:].contiguous(), mask=m2, scale=scale)
    om, lm = sd.attn_merge([o1, o2], [l1, l2])
    torch.cuda.synchronize()
    ro, rl = sdpa_fwd(f64(q), f64(k), f64(v), MASK[full], scale)
    f1 = _floor_chunk(q, k[:, :c], v[:, :c], MASK[m1], scale, DT[dtype])
    f2 = _floor_chunk(q, k[:, c:], v[:, c:], MASK[m2], scale, DT[dtype])
    fo, fl = floor_merge([f1[0], f2[0]], [f1[1], f2[1]], DT[dtype])
    _check(f"split {full} d{d} {dtype}", f64(om), lse_like_o(f64(lm), False), ro, lse_like_o(rl, False),
           fo.double().numpy(), fl.double().numpy(), dtype)


def test_split_identity_packed():
    lens = [57, 200, 131]
    c = 50  # every sequence keeps keys on both sides of the split
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    lens2 = [n - c for n in lens]
    cu1 = torch.tensor(np.concatenate([[0], np.cumsum([c] * len(lens))]), dtype=torch.int32)
    cu2 = torch.tensor(np.concatenate([[0], np.cumsum(lens2)]), dtype=torch.int32)
    t = sum(lens)
    g = torch.Generator().manual_seed(11)
    q = torch.randn(t, 4, 128, generator=g).to(torch.bfloat16)
    k = torch.randn(t, 2, 128, generator=g).to(torch.bfloat16)
    v = torch.randn(t, 2, 128, generator=g).to(torch.bfloat16)
    idx1 = torch.cat([torch.arange(int(cu[b]), int(cu[b]) + c) for b in range(len(lens))])
    idx2 = torch.cat([torch.arange(int(cu[b]) + c, int(cu[b + 1])) for b in range(len(lens))])
    qd = q.to(DEV)
    kw = dict(cu_seqlens_q=cu.to(DEV), max_seqlen_q=max(lens), scale=128 ** -0.5)
    o1, l1 = sd.attn_fwd(qd, k[idx1].to(DEV), v[idx1].to(DEV), mask="causal_tl", cu_seqlens_kv=cu1.to(DEV),
                         max_seqlen_kv=c, **kw)
    o2, l2 = sd.attn_fwd(qd, k[idx2].to(DEV), v[idx2].to(DEV), mask="causal_br", cu_seqlens_kv=cu2.to(DEV),
                         max_seqlen_kv=max(lens2), **kw)
    om, lm = sd.attn_merge([o1, o2], [l1, l2], cu_seqlens_q=cu.to(DEV), max_seqlen_q=max(lens))
    torch.cuda.synchronize()
    cun = cu.numpy()
    ro, rl = sdpa_fwd(f64(q), f64(k), f64(v), MASK_CAUSAL_TL, 128 ** -0.5, cun, cun)
    # floor: per sequence and head, each chunk in dtype, merged in dtype
    fo = torch.zeros(t, 4, 128)
    fl = torch.zeros(t, 4)
    dummy = torch.zeros(max(lens), 128, dtype=torch.bfloat16)
    for b, n in enumerate(lens):
        s0 = int(cu[b])
        for h in range(4):
            a = floor_head(q[s0:s0 + n, h], k[s0:s0 + c, h // 2], v[s0:s0 + c, h // 2], dummy[:n], 128 ** -0.5,
                           MASK_CAUSAL_TL, torch.bfloat16)
            bb = floor_head(q[s0:s0 + n, h], k[s0 + c:s0 + n, h // 2], v[s0 + c:s0 + n, h // 2], dummy[:n],
                            128 ** -0.5, MASK_CAUSAL_BR, torch.bfloat16)
            mo, ml = floor_merge([a[0].to(torch.bfloat16), bb[0].to(torch.bfloat16)], [a[1], bb[1]], torch.bfloat16)
            fo[s0:s0 + n, h] = mo
            fl[s0:s0 + n, h] = ml
    _check("split packed TL", f64(om), f64(lm), ro, rl, fo.double().numpy(), fl.double().numpy(), "bf16")


@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("split", SPLITS, ids=lambda s: s[0])
def test_ring_backward(d, split):
    full, sq, skv, c, m1, m2 = split
    dtype = "bf16"
    q, k, v, do = _inputs(sq, skv, 4, 2, d, dtype, seed=3 * d + sq)
    scale = d ** -0.5
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    k1, v1 = kd[:, :c].contiguous(), vd[:, :c].contiguous()
    k2, v2 = kd[:, c:].contiguous(), vd[:, c:].contiguous()
    o1, l1 = sd.attn_fwd(qd, k1, v1, mask=m1, scale=scale)
    o2, l2 = sd.attn_fwd(qd, k2, v2, mask=m2, scale=scale)
    om, lm = sd.attn_merge([o1, o2], [l1, l2])
    dq1, dk1, dv1 = sd.attn_bwd(qd, k1, v1, om, dod, lm, mask=m1, scale=scale)
    dq2, dk2, dv2 = sd.attn_bwd(qd, k2, v2, om, dod, lm, mask=m2, scale=scale)
    torch.cuda.synchronize()
    dq = f64(dq1) + f64(dq2)
    dk = np.concatenate([f64(dk1), f64(dk2)], axis=1)
    dv = np.concatenate([f64(dv1), f64(dv2)], axis=1)
    rdq, rdk, rdv = sdpa_bwd(f64(q), f64(k), f64(v), f64(do), MASK[full], scale)
    # single-call floor of the backward
    b_, hq, hkv = 2, 4, 2
    fdq = np.zeros_like(rdq)
    fdk = np.zeros_like(rdk)
    fdv = np.zeros_like(rdv)
    for bi in range(b_):
        for h in range(hq):
            _, _, a, bk, bv = floor_head(q[bi, :, h], k[bi, :, h // 2], v[bi, :, h // 2], do[bi, :, h], scale,
                                         MASK[full], torch.bfloat16)
            fdq[bi, :, h] = a.double().numpy()
            fdk[bi, :, h // 2] += bk.double().numpy()
            fdv[bi, :, h // 2] += bv.double().numpy()
    msgs, ok = [], True
    for name, got, ref, flo, mult in (("dQ", dq, rdq, fdq, 3.0), ("dK", dk, rdk, fdk, 2.0), ("dV", dv, rdv, fdv, 2.0)):
        err_k = float(np.abs(got - ref).max())
        err_f = float(np.abs(flo - ref).max())
        err_u = float((np.abs(got - ref) / np.maximum(1.0, np.abs(ref))).max())
        slack = 1e-6 * max(1.0, float(np.abs(ref).max()))
        good = err_u <= BOUND[dtype] and err_k <= mult * err_f + slack
        ok &= good
        msgs.append(f"{'' if good else 'FAIL '}{name}: err={err_k:.3e} floor={err_f:.3e} x{mult:g} err_u={err_u:.3e}")
    print("\n".join("    " + m for m in msgs))
    assert ok, msgs
