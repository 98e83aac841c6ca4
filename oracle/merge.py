"""Merge of attention results computed over disjoint key sets, in float64.

Test infrastructure only (see the package docstring): the product path never
imports this module.

Sources (the pages, by title and section):
  [P1] TransformerEngine pull request 3527, "cuDNN FROST attention backend for
       head_dim in (256, 512], with context parallelism", section Scope (the
       paragraph on sliding windows): the p2p (ring) context-parallel mode
       shards the keys across steps, so each step produces attention of the
       local queries over one key chunk and the steps' results are combined.
  [P3] TransformerEngine pull request 3693, "Switch to Python binding for cuDNN
       frontend", Description: empty ragged ring blocks keep neutral statistics.

Definition. For one query row let the allowed keys be the disjoint union of
chunks C_1..C_n, s_j the scaled scores and (O_k, LSE_k) attention over chunk k
alone (LSE_k = ln sum_{j in C_k} e^{s_j}). Attention over all keys is then

    LSE = ln sum_j e^{s_j} = ln sum_k e^{LSE_k}
    O   = sum_j e^{s_j - LSE} v_j = sum_k e^{LSE_k - LSE} O_k

A chunk with no allowed key for the row has LSE_k = -inf and weight 0; a row
with no allowed key in any chunk keeps O = 0 and LSE = -inf.
"""

import numpy as np


def merge(o_parts, lse_parts):
    """Combine per-chunk results of the same queries.

    o_parts: sequence of n arrays [..., D]; lse_parts: sequence of n arrays with
    the same leading shape [...] (natural-log Stats of the chunk). Returns
    (O [..., D], LSE [...]) in float64.
    """
    lse = np.stack([np.asarray(x, dtype=np.float64) for x in lse_parts])
    o = np.stack([np.asarray(x, dtype=np.float64) for x in o_parts])
    m = lse.max(axis=0)
    live = np.isfinite(m)                      # at least one chunk has a key for the row
    m0 = np.where(live, m, 0.0)
    w = np.exp(lse - m0)                       # exp(-inf) = 0: empty chunks drop out
    tot = np.where(live, w.sum(axis=0), 1.0)
    out_lse = np.where(live, m0 + np.log(tot), -np.inf)
    frac = np.where(live, w / tot, 0.0)
    out_o = (frac[..., None] * o).sum(axis=0)
    return out_o, out_lse


def lse_like_o(lse, packed):
    """Stats in the leading layout of O: dense [B, Hq, Sq] -> [B, Sq, Hq]; packed [T, Hq] unchanged."""
    lse = np.asarray(lse)
    return lse if packed else np.transpose(lse, (0, 2, 1))
