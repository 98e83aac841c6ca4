"""GPU parity: the HIP path through the C-ABI against the float64 oracle.

Two kinds of cases:
  * a sweep at sizes the oracle finishes in well under a second, spanning several
    query/key tiles with ragged tails: D in {64, 128, 256, 512} x {bf16, fp16} x
    {no mask, causal top-left, causal bottom-right} x {MHA, GQA} x {square,
    Sq < Skv, Sq > Skv (bottom-right then has empty rows)}, plus packed (THD)
    batches with lengths from 1 to 300 and unequal query/key lengths;
  * the full-size workloads (the sizes bench.py times, in the same launch
    configuration), compared on sampled (sequence, kv-head) units that the oracle
    computes one at a time. Every output buffer starts as NaN, and every element of
    every output must be written and finite, so a tile that is never written, or is
    written to another unit's place, fails even where no unit is sampled. The samples
    cover every residue of the unit index modulo 8 (the hardware deals workgroup i to
    XCD i % 8, and the launch order rotates units over XCDs and shader engines) and
    the last unit.
Acceptance is in parity_util.compare.
"""

import dataclasses
import pytest
import torch

from scaled_dot_product_02_amd.workloads import WORKLOADS, make_inputs, small

from parity_util import all_units, assert_all_written, check_units, gpu_run, run_and_check

pytestmark = pytest.mark.gpu

SHAPES = [(200, 200), (96, 333), (333, 96)]
HEADS = [(2, 2), (4, 2)]


def _sweep_cases():
    cases = []
    for d in (64, 128, 256, 512):
        for dtype in ("bf16", "fp16"):
            for mask in ("none", "causal_tl", "causal_br"):
                for sq, skv in SHAPES:
                    for hq, hkv in HEADS:
                        if d >= 256 and (hq, hkv) == (2, 2) and (sq, skv) != (200, 200):
                            continue  # keep the large-D sweep short; GQA covers the shapes
                        cases.append((d, dtype, mask, sq, skv, hq, hkv))
    return cases


@pytest.mark.parametrize("case", _sweep_cases(), ids=lambda c: "d{}-{}-{}-{}x{}-h{}_{}".format(*c))
def test_dense_sweep(case):
    d, dtype, mask, sq, skv, hq, hkv = case
    w = small(f"sweep_{d}_{dtype}_{mask}", batch=2, hq=hq, hkv=hkv, sq=sq, skv=skv, d=d, dtype=dtype, mask=mask,
              seed=d + sq)
    ok, msgs = run_and_check(w)
    assert ok, "\n".join(m for m in msgs if m.startswith("FAIL"))


THD_CASES = [
    # (lengths_q, lengths_kv or None for self-attention)
    ((1, 77, 300, 129, 64), None),
    ((50, 1, 200, 17), (120, 7, 200, 17)),
    ((130, 2, 255), (64, 300, 255)),
]


@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("mask", ["none", "causal_tl", "causal_br"])
@pytest.mark.parametrize("lens", range(len(THD_CASES)))
def test_packed_sweep(d, dtype, mask, lens):
    lq, lk = THD_CASES[lens]
    if mask != "causal_br" and lk is not None and any(a > 0 and b == 0 for a, b in zip(lq, lk)):
        pytest.skip("queries without keys are rejected for packed batches")
    w = small(f"thd_{d}_{dtype}_{mask}_{lens}", hq=4, hkv=2, d=d, dtype=dtype, mask=mask, seed=7 + lens,
              seqlens=lq, seqlens_kv=lk)
    ok, msgs = run_and_check(w)
    assert ok, "\n".join(m for m in msgs if m.startswith("FAIL"))


# Launches with more than four units per XCD (a unit count that is a multiple of 8, above 32) take each
# XCD's units four at a time: the forward and the dQ pass with more than four query tiles per unit, the
# dK/dV pass of dense batches. These cases end on partial groups (5, 9, 6 units per XCD) on the query
# side, the dK/dV side or both, and are compared whole against the oracle.
GROUPED_CASES = [
    dict(batch=5, hq=8, hkv=8, sq=640, skv=640, d=64, dtype="bf16", mask="causal_tl"),
    dict(batch=3, hq=24, hkv=8, sq=600, skv=700, d=128, dtype="fp16", mask="causal_br"),
    dict(hq=8, hkv=4, d=64, dtype="bf16", mask="causal_tl", seqlens=(700, 513, 640, 129, 900, 1)),
    dict(batch=9, hq=16, hkv=8, sq=300, skv=300, d=64, dtype="fp16", mask="none"),
    dict(batch=5, hq=16, hkv=8, sq=200, skv=200, d=512, dtype="fp16", mask="causal_tl"),  # D = 512 pair kernels
    dict(batch=6, hq=8, hkv=8, sq=700, skv=700, d=256, dtype="bf16", mask="causal_br"),
]


@pytest.mark.parametrize("case", range(len(GROUPED_CASES)))
def test_grouped_unit_order(case):
    w = small(f"grouped_{case}", seed=31 + case, **GROUPED_CASES[case])
    ok, msgs = run_and_check(w)
    assert ok, "\n".join(m for m in msgs if m.startswith("FAIL"))


# Full-size workloads: sampled units (sequence, kv-head) that the oracle computes whole. For the dense
# MHA workloads the unit index b * Hkv + g is also the query-side unit of the forward and the dQ pass;
# the samples take one unit per residue modulo 8 and the last unit.
def _residue_units(nseq, hkv, extra=()):
    """One (b, g) per residue of u = b * hkv + g modulo 8, spread over the index range, plus the last."""
    n = nseq * hkv
    picks = {n - 1, *extra}
    for r in range(8):
        if r < n:
            u = r + 8 * ((n // 8) * r // 8)  # residue r, moved further along for each r
            picks.add(min(u, n - 1 - ((n - 1 - r) % 8)))
    return sorted({(u // hkv, u % hkv) for u in picks})


FULL_UNITS = {
    "tiny": None,                   # everything
    "dense_d128": "residues",
    "thd_d128": "residues+longest+shortest",
    "dense_d512": [(0, 1), (0, 3)],  # 2 of the 4 kv-heads, the last included
    "cp_share_d256": [(0, 2), (0, 7)],
    "cp_share_d512": [(0, 3), (0, 7)],
    "window_d256": [(0, 2), (0, 7)],
    "asym_d192": [(0, 11), (1, 15)],
    "short_d128": "residues",
}


def _full_units(name, w, x):
    units = FULL_UNITS[name]
    if units is None:
        return all_units(w, x)
    if isinstance(units, list):
        return units
    nseq = len(x["seqlens_q"])
    extra = ()
    if "longest" in units:
        lens = x["seqlens_q"]
        extra = (lens.index(max(lens)) * w.hkv + 3, lens.index(min(lens)) * w.hkv + 0)
    return _residue_units(nseq, w.hkv, extra)


def test_residue_units_cover_every_xcd_and_the_last_unit():
    for nseq, hkv in ((2, 16), (16, 8), (128, 16), (1, 4), (3, 3)):
        units = _residue_units(nseq, hkv)
        idx = {b * hkv + g for b, g in units}
        assert nseq * hkv - 1 in idx
        assert {u % 8 for u in idx} == set(range(min(8, nseq * hkv)))
        assert all(0 <= b < nseq and 0 <= g < hkv for b, g in units)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_full_workload(name):
    w = WORKLOADS[name]
    x = make_inputs(w)
    print(f"full workload {name}: {w.note}", flush=True)
    got = gpu_run(w, x)
    assert_all_written(name, got)
    units = _full_units(name, w, x)
    print(f"  units compared: {units}", flush=True)
    ok, msgs = check_units(w, x, got, units)
    assert ok, "\n".join(m for m in msgs if m.startswith("FAIL"))


# Sliding windows (pull request 3527, section Scope): causal masks with a window W below the diagonal.
def _window_cases():
    cases = []
    for d in (64, 128, 256, 512):
        for dtype in ("bf16", "fp16"):
            for mask in ("causal_tl", "causal_br"):
                for wl in (0, 1, 37, 150):
                    for sq, skv in (SHAPES if d == 128 else [(200, 200)]):
                        cases.append((d, dtype, mask, wl, sq, skv))
    return cases


@pytest.mark.parametrize("case", _window_cases(), ids=lambda c: "d{}-{}-{}-w{}-{}x{}".format(*c))
def test_window_sweep(case):
    d, dtype, mask, wl, sq, skv = case
    w = small(f"win_{d}_{dtype}_{mask}_{wl}", batch=2, hq=4, hkv=2, sq=sq, skv=skv, d=d, dtype=dtype, mask=mask,
              seed=3 * d + wl + sq, window_left=wl)
    ok, msgs = run_and_check(w)
    assert ok, "\n".join(m for m in msgs if m.startswith("FAIL"))


@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("mask", ["causal_tl", "causal_br"])
@pytest.mark.parametrize("wl", [0, 37])
@pytest.mark.parametrize("lens", [0, 2])
def test_window_packed(d, mask, wl, lens):
    lq, lk = THD_CASES[lens]
    w = small(f"thdwin_{d}_{mask}_{wl}_{lens}", hq=4, hkv=2, d=d, dtype="bf16", mask=mask, seed=11 + lens,
              seqlens=lq, seqlens_kv=lk, window_left=wl)
    ok, msgs = run_and_check(w)
    assert ok, "\n".join(m for m in msgs if m.startswith("FAIL"))


@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("mask", ["causal_tl", "causal_br"])
def test_window_wider_than_every_row_is_the_causal_result_bitwise(d, mask):
    """Regression by behaviour: a window that reaches every row's first key (W >= Skv + |Skv - Sq|) must
    take the same tiles and elements as no window at all, so forward and backward agree bit for bit."""
    sq, skv = 200, 333
    w = small(f"widewin_{d}_{mask}", batch=1, hq=4, hkv=2, sq=sq, skv=skv, d=d, dtype="bf16", mask=mask, seed=23)
    x = make_inputs(w)
    a = gpu_run(w, x)
    wide = dataclasses.replace(w, window_left=skv + abs(skv - sq))
    b = gpu_run(wide, x)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[n], b[n]), n
