"""Float64 CPU oracle for fused scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call, link or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the
HIP path (no kernels, headers, helpers, tables or pre/post-processing).

What it computes is the plain definition of attention that the three pages
turn on (TransformerEngine pull request 3527, "cuDNN FROST attention backend
for head_dim in (256, 512], with context parallelism", sections Approach,
Verification and Scope; pull request 3705, section Description): scores
S = scale * Q K^T, the mask, a softmax with natural-log fp32 Stats (the
log-sum-exp), O = P V, and the gradients dQ, dK, dV. There is no tiling, no
online softmax and no rescaling: the oracle materialises S and P per head.

Modules
-------
sdpa_ref   the float64 definition (forward, backward, per-row sampling)
floor      the in-dtype computation used for the "2 x floor" criterion of
           pull request 3527, section Verification (torch CPU, fp32 math with
           every intermediate rounded to the operand dtype)
merge      the combination of attention results over disjoint key chunks
           (the p2p ring step of pull request 3527, section Scope)

Parity status of every function is pinned by tests/test_oracle_pins.py; none
is "parity unpinned" except the pages' own example values, which the pages do
not print.
"""

from .sdpa_ref import (  # noqa: F401
    MASK_NONE,
    MASK_CAUSAL_TL,
    MASK_CAUSAL_BR,
    allowed_pairs,
    head_forward,
    head_backward,
    sdpa_fwd,
    sdpa_bwd,
    count_allowed_pairs,
)
from .merge import merge, lse_like_o  # noqa: F401
