"""The in-dtype "floor" computation for the 2 x floor acceptance criterion.

Test infrastructure only (see the package docstring).

TransformerEngine pull request 3527 ("cuDNN FROST attention backend for
head_dim in (256, 512], with context parallelism"), section Verification,
states the correctness rule FlashAttention applies to itself: the kernel's
error against float64 may be at most twice the error of the same computation
done in the operand dtype, measured per case. Reading adopted here: the floor
is attention computed with operands in bf16/fp16, fp32 arithmetic, and every
intermediate tensor (S, P, O, dP, dS, dQ, dK, dV) rounded to the operand dtype
(round to nearest even, torch's conversion); the softmax statistics (row max,
LSE) and the row sums D = rowsum(dO * O) stay in fp32.

The error of rounding the inputs alone is zero here (inputs are generated in
the dtype), so that literal reading would admit no kernel at all.
"""

import torch

from .sdpa_ref import MASK_NONE, MASK_CAUSAL_TL, MASK_CAUSAL_BR


def _allowed(sq, skv, mask, window_left=-1):
    i = torch.arange(sq)[:, None]
    j = torch.arange(skv)[None, :]
    if mask == MASK_NONE:
        if window_left >= 0:
            raise ValueError("a sliding window needs a causal mask")
        return torch.ones(sq, skv, dtype=torch.bool)
    if mask == MASK_CAUSAL_TL:
        delta = 0
    elif mask == MASK_CAUSAL_BR:
        delta = skv - sq
    else:
        raise ValueError(mask)
    allow = j <= i + delta
    if window_left >= 0:
        allow = allow & (j >= i + delta - window_left)
    return allow


def floor_head(q, k, v, do, scale, mask, dtype, window_left=-1):
    """One (sequence, q-head) in dtype. Inputs are torch tensors of ``dtype``.

    Returns fp32 tensors O, LSE, dQ, dK, dV (their values are dtype-representable
    except LSE, which stays fp32).
    """
    def rnd(x):
        return x.to(dtype).to(torch.float32)

    qf, kf, vf, dof = (t.to(torch.float32) for t in (q, k, v, do))
    sq, skv = qf.shape[0], kf.shape[0]
    allow = _allowed(sq, skv, mask, window_left)
    s = rnd(scale * (qf @ kf.T))
    s = torch.where(allow, s, torch.tensor(float("-inf")))
    live = allow.any(dim=1)
    m = torch.where(live, s.max(dim=1).values, torch.zeros(sq))
    e = torch.exp(s - m[:, None])
    lse = torch.where(live, m + torch.log(e.sum(dim=1).clamp_min(1e-38)), torch.tensor(float("-inf")))
    p = rnd(torch.where(live[:, None], torch.exp(s - torch.where(live, lse, torch.zeros(sq))[:, None]), torch.zeros(sq, skv)))
    o = rnd(p @ vf)
    dp = rnd(dof @ vf.T)
    dvec = (dof * o).sum(dim=1)
    ds = rnd(p * (dp - dvec[:, None]))
    dq = rnd(scale * (ds @ kf))
    dk = rnd(scale * (ds.T @ qf))
    dv = rnd(p.T @ dof)
    return o, lse, dq, dk, dv


def floor_units(q, k, v, do, mask, scale, dtype, units, cu_seqlens_q=None, cu_seqlens_kv=None, window_left=-1):
    """Floor over the (sequence b, kv-head g) units; returns dicts keyed by unit.

    Each entry holds O and LSE for every q-head of the group ([grp, sq, D] and
    [grp, sq]) and the group-summed dK, dV ([skv, D]); per-head dK/dV are
    rounded to dtype, summed in fp32 and the sum rounded again.
    """
    hq, hkv = q.shape[-2], k.shape[-2]
    grp = hq // hkv
    out = {}
    for b, g in units:
        if cu_seqlens_q is None:
            qs, ks = (b, slice(None)), (b, slice(None))
        else:
            qs = (slice(int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])),)
            ks = (slice(int(cu_seqlens_kv[b]), int(cu_seqlens_kv[b + 1])),)
        os_, ls_, dqs = [], [], []
        dk_acc = dv_acc = None
        for h in range(g * grp, (g + 1) * grp):
            o, lse, dq, dk, dv = floor_head(q[qs + (h,)], k[ks + (g,)], v[ks + (g,)], do[qs + (h,)], scale, mask, dtype,
                                            window_left)
            os_.append(o)
            ls_.append(lse)
            dqs.append(dq)
            dk_acc = dk if dk_acc is None else dk_acc + dk
            dv_acc = dv if dv_acc is None else dv_acc + dv
        out[(b, g)] = dict(o=torch.stack(os_), lse=torch.stack(ls_), dq=torch.stack(dqs),
                           dk=dk_acc.to(dtype).to(torch.float32), dv=dv_acc.to(dtype).to(torch.float32))
    return out


def floor_merge(o_parts, lse_parts, dtype):
    """The merge of per-chunk results (oracle.merge) with fp32 arithmetic and the output O rounded to
    dtype; LSE stays fp32. o_parts: torch tensors of dtype [..., D]; lse_parts: fp32 [...].
    Returns fp32 (O, LSE)."""
    lse = torch.stack([x.to(torch.float32) for x in lse_parts])
    o = torch.stack([x.to(torch.float32) for x in o_parts])
    m = lse.max(dim=0).values
    live = torch.isfinite(m)
    m0 = torch.where(live, m, torch.zeros_like(m))
    w = torch.exp(lse - m0)
    tot = torch.where(live, w.sum(dim=0), torch.ones_like(m))
    out_lse = torch.where(live, m0 + torch.log(tot), torch.full_like(m, float("-inf")))
    frac = torch.where(live, w / tot, torch.zeros_like(w))
    out_o = (frac[..., None] * o).sum(dim=0).to(dtype).to(torch.float32)
    return out_o, out_lse
