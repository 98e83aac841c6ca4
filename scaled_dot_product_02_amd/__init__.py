"""MI355X (gfx950) fused scaled-dot-product attention engine.

The hot path (forward, backward preprocess, dK/dV pass, dQ pass) is hand-written
HIP in csrc/, behind the C-ABI of include/attn.h, built into libsdpa02.so. This
package exposes that ABI to Python under the same names (argument marshalling
only) plus the seeded synthetic workloads used by the tests and bench.py. attn_merge
combines forward results over disjoint key chunks (the ring context-parallel step).
"""

from ._binding import (  # noqa: F401
    ABI_VERSION,
    FLAG_BWD_ATOMIC_DQ,
    FLAG_FWD_EXP_SPLIT,
    FLAG_BWD_STORED_DS,
    AttnError,
    AttnProblem,
    attn_bwd,
    attn_bwd_noalloc,
    attn_bwd_workspace_bytes,
    attn_fwd,
    attn_fwd_workspace_bytes,
    attn_merge,
    attn_mfma_probe,
    attn_lds_probe,
    attn_tile_order_probe,
    lib,
    library_path,
    make_problem,
)
