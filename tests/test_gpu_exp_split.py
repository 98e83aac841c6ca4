"""GPU parity of the forward's optional exp split (ATTN_FLAG_FWD_EXP_SPLIT: on tiles without a mask, one in
four of each lane's exponentials by a VALU polynomial; head dims up to 256) against the float64 oracle,
with the acceptance of the default path (parity_util.compare), every output prefilled with NaN. The
backward runs in its default mode from the exp-split forward's O and LSE, so the check covers what a
training step with the flag would compute:
  * a dense sweep (D 64, 128, 256 x bf16/fp16 x three masks x square / Sq < Skv / Sq > Skv, GQA) at
    lengths with many interior tiles, the packed sweep, sliding windows, narrow and asymmetric heads;
  * the full-size dense D=128 workload on sampled units, every element written;
  * flag on and off agree to rounding (O within a few dtype spacings + 1e-3, LSE to 1e-5);
  * D = 512 is declined (ATTN_E_UNSUPPORTED) before any launch.
"""

import pytest
import torch

import scaled_dot_product_02_amd as sd
from scaled_dot_product_02_amd.workloads import WORKLOADS, make_inputs, small

from parity_util import assert_all_written, check_units, gpu_run, run_and_check, ulp
from test_gpu_parity import THD_CASES, _full_units

pytestmark = pytest.mark.gpu

SHAPES = [(300, 300), (200, 520), (520, 200)]


def _dense_cases():
    return [(d, dtype, mask, sq, skv) for d in (64, 128, 256) for dtype in ("bf16", "fp16")
            for mask in ("none", "causal_tl", "causal_br") for sq, skv in SHAPES]


@pytest.mark.parametrize("case", _dense_cases(), ids=lambda c: "d{}-{}-{}-{}x{}".format(*c))
def test_exp_split_dense_sweep(case):
    d, dtype, mask, sq, skv = case
    w = small(f"es_{d}_{dtype}_{mask}", batch=2, hq=4, hkv=2, sq=sq, skv=skv, d=d, dtype=dtype, mask=mask,
              seed=3 * d + sq + 7)
    ok, msgs = run_and_check(w, exp_split=True)
    assert ok, "\n".join(m for m in msgs if m.startswith("FAIL"))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", ["none", "causal_tl", "causal_br"])
@pytest.mark.parametrize("lens", range(len(THD_CASES)))
def test_exp_split_packed_sweep(d, mask, lens):
    lq, lk = THD_CASES[lens]
    if mask != "causal_br" and lk is not None and any(a > 0 and b == 0 for a, b in zip(lq, lk)):
        pytest.skip("queries without keys are rejected for packed batches")
    w = small(f"esthd_{d}_{mask}_{lens}", hq=4, hkv=2, d=d, dtype="bf16", mask=mask, seed=23 + lens,
              seqlens=lq, seqlens_kv=lk)
    ok, msgs = run_and_check(w, exp_split=True)
    assert ok, "\n".join(m for m in msgs if m.startswith("FAIL"))


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("wl", [0, 37, 150])
def test_exp_split_windows(d, wl):
    w = small(f"eswin_{d}_{wl}", batch=2, hq=4, hkv=2, sq=400, skv=400, d=d, dtype="bf16", mask="causal_br",
              seed=7 * d + wl, window_left=wl)
    ok, msgs = run_and_check(w, exp_split=True)
    assert ok, "\n".join(m for m in msgs if m.startswith("FAIL"))


@pytest.mark.parametrize("dqk,dv", [(8, 8), (40, 120), (96, 64), (192, 128), (64, 256)])
def test_exp_split_head_dims(dqk, dv):
    w = small(f"eshd_{dqk}_{dv}", batch=2, hq=4, hkv=2, sq=260, skv=330, d=dqk, dv=dv, dtype="bf16",
              mask="causal_br", seed=dqk + 5 * dv)
    ok, msgs = run_and_check(w, exp_split=True)
    assert ok, "\n".join(m for m in msgs if m.startswith("FAIL"))


def test_exp_split_full_workload():
    name = "dense_d128"
    w = WORKLOADS[name]
    x = make_inputs(w)
    print(f"full workload {name} (exp split forward): {w.note}", flush=True)
    got = gpu_run(w, x, exp_split=True)
    assert_all_written(name, got)
    units = _full_units(name, w, x)
    print(f"  units compared: {units}", flush=True)
    ok, msgs = check_units(w, x, got, units)
    assert ok, "\n".join(m for m in msgs if m.startswith("FAIL"))


def test_exp_split_agrees_with_default_and_declines_d512():
    w = small("es_agree", batch=2, hq=8, hkv=2, sq=700, skv=700, d=128, dtype="bf16", mask="causal_tl", seed=77)
    x = make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    o0, l0 = sd.attn_fwd(q, k, v, mask=w.mask, scale=w.scale)
    o1, l1 = sd.attn_fwd(q, k, v, mask=w.mask, scale=w.scale, exp_split=True)
    torch.cuda.synchronize()
    a, b = o0.double().cpu(), o1.double().cpu()
    # the row sums take the polynomial's values unrounded: some LSE must differ in its last bits
    assert not torch.equal(l0, l1), "the flag changed nothing: the split path did not run"
    # a P value whose bf16 rounding flips moves O by up to 2^-8 of that P's share: a few spacings, plus an
    # absolute term for outputs near zero (both sides are held to the oracle by the tests above)
    lim = 4 * torch.from_numpy(ulp(a.numpy(), "bf16")) + 1e-3
    assert ((a - b).abs() <= lim).all(), float((a - b).abs().max())
    assert (l0 - l1).abs().max().item() < 1e-5
    q5 = torch.zeros(1, 64, 2, 512, dtype=torch.bfloat16, device=dev)
    with pytest.raises(sd.AttnError) as e:
        sd.attn_fwd(q5, q5, q5, exp_split=True)
    assert e.value.status_name == "ATTN_E_UNSUPPORTED"
