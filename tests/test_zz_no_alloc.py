"""GPU: attn_bwd_noalloc (the backward on the library's own scratch array, for callers that cannot
allocate) against attn_bwd with a caller workspace, through the C-ABI.

Two calls in a row, the second with a smaller (packed) input, so the second runs on an array that
still holds the first call's contents: both must equal attn_bwd bit for bit (the same kernels on the
same inputs) and meet the oracle bar of the parity tests. A problem larger than the array is declined
before any launch (checked on the CPU in the contract tests too).
"""

import pytest
import torch

import scaled_dot_product_02_amd as sd
from scaled_dot_product_02_amd.workloads import make_inputs, small

from parity_util import check_units, all_units

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _inputs(w):
    x = make_inputs(w)
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    kw = dict(mask=w.mask, scale=w.scale, window_left=w.window_left)
    if w.packed:
        kw.update(cu_seqlens_q=x["cu_seqlens_q"].to(DEV), cu_seqlens_kv=x["cu_seqlens_kv"].to(DEV),
                  max_seqlen_q=x["max_seqlen_q"], max_seqlen_kv=x["max_seqlen_kv"])
    return x, q, k, v, do, kw


def _nan(t):
    return torch.full_like(t, float("nan"))


def test_noalloc_matches_attn_bwd_on_two_calls_the_second_smaller():
    cases = [
        small("noalloc_big", batch=2, hq=8, hkv=2, sq=700, skv=700, d=128, dtype="bf16", mask="causal_tl", seed=41),
        small("noalloc_small", hq=4, hkv=2, d=64, dtype="fp16", mask="causal_br", seed=42, seqlens=(40, 1, 77),
              seqlens_kv=(60, 5, 77)),
    ]
    for w in cases:
        print(f"noalloc case {w.name}", flush=True)
        x, q, k, v, do, kw = _inputs(w)
        o, lse = sd.attn_fwd(q, k, v, **kw)
        ref = sd.attn_bwd(q, k, v, o, do, lse, dq=_nan(q), dk=_nan(k), dv=_nan(v), **kw)
        got = sd.attn_bwd_noalloc(q, k, v, o, do, lse, dq=_nan(q), dk=_nan(k), dv=_nan(v), **kw)
        torch.cuda.synchronize()
        for n, a, b in zip(("dQ", "dK", "dV"), ref, got):
            assert torch.isfinite(b).all(), f"{w.name}: {n} has unwritten elements"
            assert torch.equal(a, b), f"{w.name}: attn_bwd_noalloc differs from attn_bwd in {n}"
        res = dict(o=o.cpu(), lse=lse.cpu(), dq=got[0].cpu(), dk=got[1].cpu(), dv=got[2].cpu())
        ok, msgs = check_units(w, x, res, all_units(w, x))
        assert ok, "\n".join(m for m in msgs if m.startswith("FAIL"))


def test_noalloc_stored_ds_matches_attn_bwd():
    """The stored-dS backward on the library's array (its dS lives there too): two calls in a row, the second
    smaller and packed, each equal to attn_bwd with the flag and a caller workspace, bit for bit."""
    cases = [
        small("noalloc_sds_big", batch=1, hq=4, hkv=2, sq=300, skv=300, d=512, dtype="bf16", mask="causal_tl",
              seed=43),
        small("noalloc_sds_small", hq=2, hkv=1, d=264, dv=512, dtype="fp16", mask="causal_br", seed=44,
              seqlens=(40, 1, 77), seqlens_kv=(60, 5, 77)),
    ]
    for w in cases:
        print(f"noalloc stored-dS case {w.name}", flush=True)
        x, q, k, v, do, kw = _inputs(w)
        o, lse = sd.attn_fwd(q, k, v, **kw)
        ref = sd.attn_bwd(q, k, v, o, do, lse, dq=_nan(q), dk=_nan(k), dv=_nan(v), stored_ds=True, **kw)
        got = sd.attn_bwd_noalloc(q, k, v, o, do, lse, dq=_nan(q), dk=_nan(k), dv=_nan(v), stored_ds=True, **kw)
        torch.cuda.synchronize()
        for n, a, b in zip(("dQ", "dK", "dV"), ref, got):
            assert torch.isfinite(b).all(), f"{w.name}: {n} has unwritten elements"
            assert torch.equal(a, b), f"{w.name}: attn_bwd_noalloc differs from attn_bwd in {n}"


def test_noalloc_declines_problems_beyond_its_array():
    # 2 x 262144 query rows x 8 heads x 8 bytes = 32 MiB of row arrays, beyond the 16 MiB array
    q = torch.empty(2, 262144, 8, 64, dtype=torch.bfloat16, device=DEV)
    k = torch.empty(2, 64, 8, 64, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(2, 8, 262144, dtype=torch.float32, device=DEV)
    with pytest.raises(sd.AttnError) as e:
        sd.attn_bwd_noalloc(q, k, k, q, q, lse)
    assert e.value.status_name == "ATTN_E_WORKSPACE" and "attn_bwd_noalloc" in e.value.reason
