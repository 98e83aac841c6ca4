"""Shared helpers for the GPU parity tests (not a test module).

Acceptance per case and output tensor (pull request 3527, section Verification:
the kernel's error against float64 may be at most twice the error of the same
computation in the operand dtype, measured per case), plus the fixed bounds of
this engine's target: 2e-2 (bf16) / 5e-3 (fp16) on O, dQ, dK, dV and 1e-3 on LSE.

* 2 x floor: err = max |kernel - ref| over the compared elements, against the
  same for the floor. When the floor is exact (err_f = 0) a slack of
  1e-6 * max(1, max|ref|) stands in for 2 * err_f.
* fixed bound: max |kernel - ref| / max(1, |ref|), elementwise, i.e. absolute
  error where |ref| <= 1 and relative error above. Reading: an absolute bound
  cannot be the intent for outputs larger than ~10, because rounding the exact
  result to bf16 alone then exceeds 2e-2 (half an ulp of a value in [8, 16) is
  2^-5 = 0.031; GQA dV sums reach that size); in units of max(1, |ref|) the
  output rounding is at most 2^-9 (bf16) / 2^-12 (fp16).
Rows whose oracle LSE is -inf (no allowed key) must be -inf exactly and are
left out of the LSE errors.
"""

import time

import numpy as np
import torch

import scaled_dot_product_02_amd as sd
from oracle import floor as oracle_floor
from oracle import sdpa_bwd, sdpa_fwd
from scaled_dot_product_02_amd.workloads import make_inputs

MASK_TO_ORACLE = {"none": 0, "causal_tl": 1, "causal_br": 2}
BOUND = {"bf16": 2e-2, "fp16": 5e-3}


def f64(t):
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def gpu_run(w, x, backward=True, stream=None):
    """Forward (and backward) of workload w on cuda:0 through the C-ABI; returns CPU tensors."""
    dev = torch.device("cuda:0")
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    kw = dict(mask=w.mask, scale=w.scale, window_left=w.window_left)
    if w.packed:
        kw.update(cu_seqlens_q=x["cu_seqlens_q"].to(dev), cu_seqlens_kv=x["cu_seqlens_kv"].to(dev),
                  max_seqlen_q=x["max_seqlen_q"], max_seqlen_kv=x["max_seqlen_kv"])
    o, lse = sd.attn_fwd(q, k, v, stream=stream, **kw)
    out = dict(o=o, lse=lse)
    if backward:
        do = x["do"].to(dev)
        dq, dk, dv = sd.attn_bwd(q, k, v, o, do, lse, stream=stream, **kw)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {n: t.cpu() for n, t in out.items()}


def _unit_views(w, x, b, g):
    """Index helpers for one (sequence b, kv-head g) unit: returns (q_rows, kv_rows, heads) selectors."""
    grp = w.hq // w.hkv
    heads = list(range(g * grp, (g + 1) * grp))
    if w.packed:
        cq, ck = x["cu_seqlens_q"], x["cu_seqlens_kv"]
        qs = slice(int(cq[b]), int(cq[b + 1]))
        ks = slice(int(ck[b]), int(ck[b + 1]))
    else:
        qs = ks = None
    return qs, ks, heads


def _take_q(w, t, b, qs, heads):
    """[grp, rows, D] (or [grp, rows] for LSE) of a q-side tensor for one unit."""
    if w.packed:
        return np.stack([t[qs, h] for h in heads])
    return np.stack([t[b, :, h] for h in heads])


def _take_lse(w, t, b, qs, heads):
    if w.packed:
        return np.stack([t[qs, h] for h in heads])
    return np.stack([t[b, h] for h in heads])


def _take_kv(w, t, b, ks, g):
    return t[ks, g] if w.packed else t[b, :, g]


def compare(name, got, ref, flo, dtype, is_lse=False):
    """Returns (ok, message) for one tensor under both criteria."""
    if is_lse:
        live = np.isfinite(ref)
        if not np.array_equal(np.isneginf(got), ~live):
            return False, f"{name}: -inf pattern differs from the oracle"
        got, ref, flo = got[live], ref[live], flo[live]
    if got.size == 0:
        return True, f"{name}: empty"
    if not np.isfinite(got).all():
        return False, f"{name}: non-finite values"
    err_k = float(np.abs(got - ref).max())
    err_f = float(np.abs(flo - ref).max())
    err_u = float((np.abs(got - ref) / np.maximum(1.0, np.abs(ref))).max())
    bound = 1e-3 if is_lse else BOUND[dtype]
    slack = 1e-6 * max(1.0, float(np.abs(ref).max()))
    ok = err_u <= bound and err_k <= 2 * err_f + slack
    rel_rms = float(np.sqrt(np.mean((got - ref) ** 2)) / max(np.sqrt(np.mean(ref ** 2)), 1e-30))
    return ok, (f"{name}: err={err_k:.3e} floor={err_f:.3e} ratio={err_k / max(err_f, 1e-30):.2f} "
                f"err/max(1,|ref|)={err_u:.3e} bound={bound:.0e} relrms={rel_rms:.2e}")


def check_units(w, x, got, units, verbose=True):
    """Compare GPU outputs with the float64 oracle and the in-dtype floor on the given units."""
    mask = MASK_TO_ORACLE[w.mask]
    t0 = time.time()
    xin = {n: f64(x[n]) for n in ("q", "k", "v", "do")}
    cu_q = x["cu_seqlens_q"].numpy() if w.packed else None
    cu_k = x["cu_seqlens_kv"].numpy() if w.packed else None
    ro, rl = sdpa_fwd(xin["q"], xin["k"], xin["v"], mask, w.scale, cu_q, cu_k, units=units,
                      window_left=w.window_left)
    rdq, rdk, rdv = sdpa_bwd(xin["q"], xin["k"], xin["v"], xin["do"], mask, w.scale, cu_q, cu_k, units=units,
                             window_left=w.window_left)
    t1 = time.time()
    flo = oracle_floor.floor_units(x["q"], x["k"], x["v"], x["do"], mask, w.scale, w.torch_dtype, units,
                                   x["cu_seqlens_q"], x["cu_seqlens_kv"], window_left=w.window_left)
    t2 = time.time()
    g64 = {n: f64(t) for n, t in got.items()}
    msgs, all_ok = [], True
    for (b, g) in units:
        qs, ks, heads = _unit_views(w, x, b, g)
        fl = flo[(b, g)]
        pairs = [
            ("O", _take_q(w, g64["o"], b, qs, heads), _take_q(w, ro, b, qs, heads), fl["o"].double().numpy(), False),
            ("LSE", _take_lse(w, g64["lse"], b, qs, heads), _take_lse(w, rl, b, qs, heads),
             fl["lse"].double().numpy(), True),
        ]
        if "dq" in got:
            pairs += [
                ("dQ", _take_q(w, g64["dq"], b, qs, heads), _take_q(w, rdq, b, qs, heads),
                 fl["dq"].double().numpy(), False),
                ("dK", _take_kv(w, g64["dk"], b, ks, g), _take_kv(w, rdk, b, ks, g), fl["dk"].double().numpy(), False),
                ("dV", _take_kv(w, g64["dv"], b, ks, g), _take_kv(w, rdv, b, ks, g), fl["dv"].double().numpy(), False),
            ]
        for name, gv, rv, fv, is_lse in pairs:
            ok, m = compare(f"unit{(b, g)} {name}", gv, rv, fv, w.dtype, is_lse)
            all_ok &= ok
            msgs.append(("" if ok else "FAIL ") + m)
    if verbose:
        print(f"[{w.name}] oracle {t1 - t0:.1f}s floor {t2 - t1:.1f}s")
        for m in msgs:
            print("   ", m)
    return all_ok, msgs


def all_units(w, x):
    nseq = len(x["seqlens_q"]) if w.packed else w.batch
    return [(b, g) for b in range(nseq) for g in range(w.hkv)]


def run_and_check(w, units=None, backward=True):
    x = make_inputs(w)
    got = gpu_run(w, x, backward=backward)
    return check_units(w, x, got, units if units is not None else all_units(w, x))
