"""The float64 definition of scaled-dot-product attention, forward and backward.

Test infrastructure only (see the package docstring): the product path never
imports this module.

Sources (the pages, by title and section):
  [P1] TransformerEngine pull request 3527, "cuDNN FROST attention backend for
       head_dim in (256, 512], with context parallelism".
       - Approach: the all-gather path turns a causal mask into a
         bottom-right-aligned causal band on the trimmed KV range.
       - Verification: forward, the LSE convention and the gradients are
         checked against an independent float64 reference; coverage is
         square and rectangular shapes, causal / bottom-right / no mask, GQA
         and MHA.
       - Scope: the mask vocabulary no_mask / causal / causal_bottom_right;
         head dims: the backward engine there is declared for any multiple
         of 8 up to 512 (padded to its compiled width) and is held to
         d_qk == d_v only by an engine flag, while the forward engine lists
         the asymmetric pair (192, 128) natively.
  [P2] TransformerEngine pull request 3705 (FROST forward provider for
       context-parallel attention), section Description / Execution and
       supported scope: the forward returns fp32 Stats that are natural
       logarithms, token-major for packed (THD) batches, and the backward
       consumes them; packed batches are described by zero-based cumulative
       sequence lengths with no holes.
  [P3] TransformerEngine pull request 3693, "Switch to Python binding for cuDNN
       frontend", review comments on the PyTorch fused-attention wrapper: the
       Stats tensor is [tq, h, 1] for packed thd inputs and [b, h, sq, 1] for
       bshd/sbhd; the attention scale is an fp32 scalar passed by value.

Readings where the pages are silent:
  * causal top-left (TL): key j is allowed for query i iff j <= i.
    causal bottom-right (BR): j <= i + (Skv - Sq), per sequence.  [P1 Approach,
    Scope name both; the diagonals are the standard ones, pinned by the TL==BR
    and context-parallel-share identities in the tests.]
  * GQA: q-head h reads kv-head h // (Hq // Hkv) (contiguous groups).
  * A query row with no allowed key has O = 0, LSE = -inf and zero gradient
    (neutral statistics; [P3] Description mentions neutral statistics for empty
    ragged ring blocks).
  * The scale multiplies Q K^T before masking and softmax.
  * Head dims: Q and K share D_qk, V and O (hence dO, dV) have their own
    D_v; nothing else depends on either (the scale is passed by value), so
    the definition below is the same for any pair.  [P1 Scope; pinned by the
    V-column split and zero-padding identities and by finite differences.]

Layouts: dense Q is [B, Sq, Hq, D_qk], O/dO [B, Sq, Hq, D_v], K [B, Skv, Hkv,
D_qk], V [B, Skv, Hkv, D_v]; packed (THD) drops the batch axis and uses the
token axis ([Tq, ...], [Tkv, ...]) with cu_seqlens of length B+1.
LSE is [B, Hq, Sq] dense and [Tq, Hq] packed (token-major).
"""

import numpy as np

MASK_NONE = 0
MASK_CAUSAL_TL = 1
MASK_CAUSAL_BR = 2


def allowed_pairs(sq, skv, mask, window_left=-1):
    """Boolean [sq, skv]: which (query, key) pairs the mask admits.

    [P1] Scope names the three masks; [P1] Approach describes the
    bottom-right band (the causal diagonal aligned to the last key). With
    window_left = W >= 0 a causal mask also drops keys more than W before the
    diagonal ([P1] Scope, sliding windows).
    """
    i = np.arange(sq)[:, None]
    j = np.arange(skv)[None, :]
    if mask == MASK_NONE:
        if window_left >= 0:
            raise ValueError("a sliding window needs a causal mask (it fixes the diagonal)")
        return np.ones((sq, skv), dtype=bool)
    if mask == MASK_CAUSAL_TL:
        delta = 0
    elif mask == MASK_CAUSAL_BR:
        delta = skv - sq
    else:
        raise ValueError(f"unknown mask {mask}")
    allow = j <= i + delta
    if window_left >= 0:
        allow &= j >= i + delta - window_left
    return allow


def head_forward(q, k, v, scale, mask, window_left=-1):
    """One (sequence, q-head): returns O [sq, D_v], LSE [sq] (natural log), P [sq, skv].

    S = scale * q k^T; masked entries are -inf; LSE_i = log sum_j exp(S_ij)
    (natural log, [P2] Description); P_ij = exp(S_ij - LSE_i); O = P v.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    sq, skv = q.shape[0], k.shape[0]
    allow = allowed_pairs(sq, skv, mask, window_left)
    s = np.where(allow, scale * (q @ k.T), -np.inf)
    live = allow.any(axis=1)
    lse = np.full(sq, -np.inf)
    p = np.zeros((sq, skv))
    if live.any():
        sl = s[live]
        m = sl.max(axis=1)
        lse[live] = m + np.log(np.exp(sl - m[:, None]).sum(axis=1))
        p[live] = np.exp(sl - lse[live][:, None])
    o = p @ v
    return o, lse, p


def head_backward(q, k, v, do, scale, mask, window_left=-1):
    """One (sequence, q-head): returns dQ [sq, D_qk], dK [skv, D_qk], dV [skv, D_v].

    Gradients of the forward above with respect to q, k, v for the upstream
    gradient dO ([P1] Verification checks exactly these against float64):
      dV = P^T dO
      dP = dO v^T
      D_i = sum_j P_ij dP_ij
      dS = P * (dP - D)
      dQ = scale * dS k
      dK = scale * dS^T q
    Rows with no allowed key have P = 0 and so contribute nothing.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    _, _, p = head_forward(q, k, v, scale, mask, window_left)
    dv = p.T @ do
    dp = do @ v.T
    dvec = (p * dp).sum(axis=1)
    ds = p * (dp - dvec[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def _sequences(q, k, cu_seqlens_q, cu_seqlens_kv):
    """Yield (b, q_index, kv_index) where the indices select one sequence's rows.

    Dense: q[b], k[b] (index tuples into the leading axes).
    Packed: rows cu[b]:cu[b+1] of the token axis ([P2] Execution and supported
    scope: zero-based cumulative lengths, no holes).
    """
    if cu_seqlens_q is None:
        for b in range(q.shape[0]):
            yield b, (b, slice(None)), (b, slice(None))
    else:
        cq = np.asarray(cu_seqlens_q, dtype=np.int64)
        ck = np.asarray(cu_seqlens_kv, dtype=np.int64)
        for b in range(len(cq) - 1):
            yield b, (slice(int(cq[b]), int(cq[b + 1])),), (slice(int(ck[b]), int(ck[b + 1])),)


def _check(q, k, v, packed):
    hq, hkv = q.shape[-2], k.shape[-2]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if v.shape[:-1] != k.shape[:-1]:
        raise ValueError("K and V must have the same tokens and heads")
    if q.shape[-1] != k.shape[-1]:
        raise ValueError("Q and K head dims differ")
    if (q.ndim != 3) if packed else (q.ndim != 4):
        raise ValueError("dense tensors are [B,S,H,D]; packed tensors are [T,H,D]")
    return hq, hkv


def _units(nseq, hkv, units):
    return [(b, g) for b in range(nseq) for g in range(hkv)] if units is None else list(units)


def sdpa_fwd(q, k, v, mask, scale, cu_seqlens_q=None, cu_seqlens_kv=None, units=None, window_left=-1):
    """Forward over a batch: returns O (float64, Q's layout with V's head dim) and LSE.

    ``units`` optionally restricts the work to (sequence b, kv-head g) pairs;
    every q-head of g's group is computed there, and all other outputs are NaN.
    LSE is [B, Hq, Sq] dense and [Tq, Hq] packed ([P3] review comments on the
    Stats layouts; [P2] token-major packed Stats).
    """
    packed = cu_seqlens_q is not None
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    hq, hkv = _check(q, k, v, packed)
    grp = hq // hkv
    o = np.full(q.shape[:-1] + v.shape[-1:], np.nan)
    lse = np.full(q.shape[:-1], np.nan) if packed else np.full((q.shape[0], hq, q.shape[1]), np.nan)
    seqs = list(_sequences(q, k, cu_seqlens_q, cu_seqlens_kv))
    for b, g in _units(len(seqs), hkv, units):
        _, qi, ki = seqs[b]
        for h in range(g * grp, (g + 1) * grp):
            oh, lh, _ = head_forward(q[qi + (h,)], k[ki + (g,)], v[ki + (g,)], scale, mask, window_left)
            o[qi + (h,)] = oh
            if packed:
                lse[qi + (h,)] = lh
            else:
                lse[b, h] = lh
    return o, lse


def sdpa_bwd(q, k, v, do, mask, scale, cu_seqlens_q=None, cu_seqlens_kv=None, units=None, window_left=-1):
    """Backward over a batch: returns dQ, dK, dV (float64, layouts of Q, K, V).

    dK and dV of kv-head g sum the contributions of every q-head in g's group.
    ``units`` as in sdpa_fwd.
    """
    packed = cu_seqlens_q is not None
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    hq, hkv = _check(q, k, v, packed)
    if do.shape != q.shape[:-1] + v.shape[-1:]:
        raise ValueError("dO must have O's shape (Q's layout with V's head dim)")
    grp = hq // hkv
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    seqs = list(_sequences(q, k, cu_seqlens_q, cu_seqlens_kv))
    for b, g in _units(len(seqs), hkv, units):
        _, qi, ki = seqs[b]
        dk_acc = np.zeros(k[ki + (g,)].shape)
        dv_acc = np.zeros(v[ki + (g,)].shape)
        for h in range(g * grp, (g + 1) * grp):
            dqh, dkh, dvh = head_backward(q[qi + (h,)], k[ki + (g,)], v[ki + (g,)], do[qi + (h,)], scale, mask,
                                          window_left)
            dq[qi + (h,)] = dqh
            dk_acc += dkh
            dv_acc += dvh
        dk[ki + (g,)] = dk_acc
        dv[ki + (g,)] = dv_acc
    return dq, dk, dv


def count_allowed_pairs(seqlens_q, seqlens_kv, mask, window_left=-1):
    """Number of allowed (query, key) pairs summed over sequences, for one head.

    Closed forms of the masks above: none -> Sq*Skv; causal with diagonal
    delta (0 for TL, Skv - Sq for BR): row i sees keys max(0, i + delta - W)
    .. min(Skv - 1, i + delta), i.e. clip(i + delta + 1, 0, Skv) keys less the
    clip(i + delta - W, 0, Skv) keys before the window (W = -1: none).
    """
    total = 0
    for sq, skv in zip(seqlens_q, seqlens_kv):
        sq, skv = int(sq), int(skv)
        i = np.arange(sq, dtype=np.int64)
        if mask == MASK_NONE:
            if window_left >= 0:
                raise ValueError("a sliding window needs a causal mask (it fixes the diagonal)")
            total += sq * skv
            continue
        if mask == MASK_CAUSAL_TL:
            delta = 0
        elif mask == MASK_CAUSAL_BR:
            delta = skv - sq
        else:
            raise ValueError(f"unknown mask {mask}")
        upto = np.clip(i + delta + 1, 0, skv)
        before = np.clip(i + delta - window_left, 0, skv) if window_left >= 0 else 0
        total += int(np.maximum(upto - before, 0).sum())
    return total
