"""GPU checks at the largest sizes the interface takes: tensors of more than 2^31 elements (every
address is formed in 64 bits) and a sequence of 2^20 tokens. Forward and backward run in full on the
GPU; the float64 oracle checks the tail: the last TAIL query rows of the last heads (O, LSE, dQ) and
the last TAIL keys (dK, dV).

Why the tail can be checked alone (TransformerEngine pull request 3527, section Scope, mask vocabulary):
under a top-left causal mask query row i of a sequence of S tokens sees keys 0..i, so the last TAIL rows
are the bottom-right causal problem of TAIL rows against all S keys; and key j receives gradient only
from rows i >= j, so for the last TAIL keys every contributing row is in the tail. Inputs are drawn on
the GPU by torch's seeded generator (too large to draw on the host); the slices the oracle reads are
copied back. Bounds: the fixed ones of the parity tests (bf16: |err| <= max(2e-2, one bf16 spacing at
|ref|) elementwise on O and the gradients, 1e-3 absolute on LSE); every element of every output must be
finite.
"""

import numpy as np
import pytest
import torch

import scaled_dot_product_02_amd as sd
from oracle import MASK_CAUSAL_BR, head_backward, head_forward
from scaled_dot_product_02_amd.workloads import draw_device

from parity_util import fixed_bound

pytestmark = pytest.mark.gpu


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _run_and_check_tail(B, S, H, D, tail, heads, seed):
    dev = torch.device("cuda:0")
    dt = torch.bfloat16
    shape = (B, S, H, D)
    q, k, v, do = (draw_device(shape, seed + i, dt, dev) for i in range(4))
    scale = 1.0 / D ** 0.5
    print(f"large case B{B} S{S} H{H} D{D}: {q.numel()} elements per tensor", flush=True)
    o, lse = sd.attn_fwd(q, k, v, mask="causal_tl", scale=scale)
    dq, dk, dv = sd.attn_bwd(q, k, v, o, do, lse, mask="causal_tl", scale=scale)
    torch.cuda.synchronize()
    for n, t in (("O", o), ("dQ", dq), ("dK", dk), ("dV", dv), ("LSE", lse)):
        assert bool(torch.isfinite(t).all()), f"{n}: non-finite elements"
    b = B - 1
    tr = slice(S - tail, S)
    worst = {}
    for h in heads:
        qs, dos = _f64(q[b, tr, h]), _f64(do[b, tr, h])
        kf, vf = _f64(k[b, :, h]), _f64(v[b, :, h])
        ro, rl, _ = head_forward(qs, kf, vf, scale, MASK_CAUSAL_BR)
        rdq, rdk, rdv = head_backward(qs, kf, vf, dos, scale, MASK_CAUSAL_BR)
        pairs = [("O", _f64(o[b, tr, h]), ro), ("dQ", _f64(dq[b, tr, h]), rdq),
                 ("dK", _f64(dk[b, tr, h]), rdk[S - tail:]), ("dV", _f64(dv[b, tr, h]), rdv[S - tail:])]
        for name, got, ref in pairs:
            err = float((np.abs(got - ref) / fixed_bound(ref, "bf16")).max())  # <= 1 passes
            worst[name] = max(worst.get(name, 0.0), err)
        err_l = float(np.abs(lse[b, h, tr].cpu().numpy().astype(np.float64) - rl).max())
        worst["LSE"] = max(worst.get("LSE", 0.0), err_l)
    print("worst errors (LSE absolute, others as a fraction of their bound):",
          {n: f"{e:.2e}" for n, e in worst.items()}, flush=True)
    for name, e in worst.items():
        assert e <= (1e-3 if name == "LSE" else 1.0), (name, e)


def test_tensors_beyond_2g_elements():
    # 2 x 65536 x 128 x 128 = 2^31 elements per tensor (4 GiB in bf16): element offsets past int32
    B, S, H, D = 2, 65536, 128, 128
    assert B * S * H * D >= 2 ** 31
    _run_and_check_tail(B, S, H, D, tail=64, heads=(H - 2, H - 1), seed=101)


def test_sequence_of_2_20_tokens():
    _run_and_check_tail(1, 2 ** 20, 2, 128, tail=32, heads=(1,), seed=111)
