"""GPU: the backward's separate entry points against attn_bwd and the float64 oracle.

attn_bwd runs the dQ pass with the preprocess folded in, then the dK/dV pass, for head
dims up to 256, and preprocess, dK/dV, dQ for wider heads. Each order a caller may use is
checked here on the same inputs:
  * "dq_preprocess" then "dkdv" gives attn_bwd's outputs bit for bit (the same launches);
  * "preprocess", "dkdv", "dq" (the three-pass order) meets the oracle bar on its own:
    the folded preprocess sums O*dO in another order, so the two orders may differ by
    rounding, not by more;
  * "preprocess" then "dq_preprocess" then "dkdv" (the preprocess run twice) also agrees.
Dense cases include bottom-right causal with Sq > Skv, whose first rows have no key:
their LSE is -inf and the folded preprocess must hand the dK/dV pass +inf, as the
standalone preprocess does, so those rows add nothing to dK/dV.
"""

import pytest
import torch

import scaled_dot_product_02_amd as sd
from scaled_dot_product_02_amd.workloads import make_inputs, small

from parity_util import all_units, check_units

pytestmark = pytest.mark.gpu

ORDERS = {
    "fused": ("dq_preprocess", "dkdv"),
    "split": ("preprocess", "dkdv", "dq"),
    "split_dq_first": ("preprocess", "dq", "dkdv"),
    "twice": ("preprocess", "dq_preprocess", "dkdv"),
}


def _run_orders(w, x):
    dev = torch.device("cuda:0")
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    kw = dict(mask=w.mask, scale=w.scale, window_left=w.window_left)
    if w.packed:
        kw.update(cu_seqlens_q=x["cu_seqlens_q"].to(dev), cu_seqlens_kv=x["cu_seqlens_kv"].to(dev),
                  max_seqlen_q=x["max_seqlen_q"], max_seqlen_kv=x["max_seqlen_kv"])
    o, lse = sd.attn_fwd(q, k, v, **kw)
    res = {"all": sd.attn_bwd(q, k, v, o, do, lse, **kw)}
    for name, passes in ORDERS.items():
        # fresh outputs filled with NaN, so an element a pass order fails to write shows up
        outs = {n: torch.full_like(t, float("nan")) for n, t in zip(("dq", "dk", "dv"), (q, k, v))}
        res[name] = sd.attn_bwd(q, k, v, o, do, lse, passes=passes, **outs, **kw)
    torch.cuda.synchronize()
    fwd = dict(o=o.cpu(), lse=lse.cpu())
    return fwd, {name: [t.cpu() for t in r] for name, r in res.items()}


def _check(w):
    x = make_inputs(w)
    fwd, res = _run_orders(w, x)
    wide = max(w.d, w.d_v) > 256
    same_as_all = ("split", "split_dq_first") if wide else ("fused", "twice")
    for name in same_as_all:
        for n, a, b in zip(("dQ", "dK", "dV"), res["all"], res[name]):
            assert torch.equal(a, b), f"{w.name}: passes {ORDERS[name]} differ from attn_bwd in {n}"
    for name in ("all",) + tuple(ORDERS):
        got = dict(fwd, dq=res[name][0], dk=res[name][1], dv=res[name][2])
        ok, msgs = check_units(w, x, got, all_units(w, x), verbose=False)
        assert ok, f"{w.name} passes {name}:\n" + "\n".join(m for m in msgs if m.startswith("FAIL"))


@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("mask,sq,skv", [("causal_br", 333, 96), ("causal_tl", 200, 200), ("none", 96, 333)])
def test_pass_orders_dense(d, mask, sq, skv):
    _check(small(f"passes_{d}_{mask}", batch=2, hq=4, hkv=2, sq=sq, skv=skv, d=d, dtype="bf16", mask=mask,
                 seed=11 + d))


@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("mask", ["causal_tl", "causal_br"])
def test_pass_orders_packed(d, mask):
    _check(small(f"passes_thd_{d}_{mask}", hq=4, hkv=2, d=d, dtype="fp16", mask=mask, seed=5 + d,
                 seqlens=(50, 1, 200, 17), seqlens_kv=(120, 7, 200, 17)))


def test_pass_orders_window_asym():
    """A sliding window with Q/K head dim 192 and V head dim 128 (the folded preprocess reads O at D_v)."""
    _check(small("passes_window_asym", batch=2, hq=4, hkv=1, sq=300, skv=300, d=192, dv=128, dtype="bf16",
                 mask="causal_tl", seed=3, window_left=100))
