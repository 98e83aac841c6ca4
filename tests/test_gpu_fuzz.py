"""GPU parity on seeded random configurations: the HIP path through the C-ABI against the float64
oracle, on shapes the fixed sweeps do not pin down. Each case draws, from one fixed seed, a head dim
(any multiple of 8 up to 512, Q/K and V/O equal or not), dtype, mask (none, causal top-left, causal
bottom-right; causal masks with or without a sliding window), MHA or GQA, and either a dense batch with
independent query and key lengths (1 .. 500, so bottom-right cases with more queries than keys have
empty rows) or a packed batch of 1-4 sequences with lengths 0 .. 400 (empty sequences included).
Acceptance is parity_util.compare (2 x floor and the fixed bounds), every output NaN-prefilled and
required to be written. The configurations with a head above 256 also run through the stored-dS backward.
"""

import numpy as np
import pytest

from parity_util import run_and_check
from scaled_dot_product_02_amd.workloads import small

pytestmark = pytest.mark.gpu

N_CASES = 120
WORK_LIMIT = 2e8  # heads x Sq x Skv x max head dim: keeps every oracle run to seconds


def _cases():
    rng = np.random.RandomState(20261202)
    out = []
    for i in range(N_CASES):
        d = 8 * int(rng.randint(1, 65))
        dv = d if rng.rand() < 0.7 else 8 * int(rng.randint(1, 65))
        dtype = str(rng.choice(["bf16", "fp16"]))
        mask = str(rng.choice(["none", "causal_tl", "causal_br"]))
        wl = int(rng.choice([-1, -1, 0, 5, 64, 200])) if mask != "none" else -1
        hkv = int(rng.randint(1, 4))
        hq = hkv * int(rng.choice([1, 2, 4]))
        kw = dict(hq=hq, hkv=hkv, d=d, dv=dv, dtype=dtype, mask=mask, window_left=wl, seed=1000 + i)
        dmax = max(d, dv)
        if rng.rand() < 0.35:
            n = int(rng.randint(1, 5))
            lq = rng.randint(0, 401, n)
            lk = lq.copy() if rng.rand() < 0.5 else rng.randint(0, 401, n)
            if mask != "causal_br":
                lk = np.where((lq > 0) & (lk == 0), 1, lk)  # queries without keys are declined there
            while hq * int((lq * lk).sum()) * dmax > WORK_LIMIT:
                lq, lk = lq // 2, np.where(lk > 1, lk // 2, lk)
            kw.update(seqlens=[int(x) for x in lq], seqlens_kv=[int(x) for x in lk])
        else:
            b = int(rng.randint(1, 3))
            sq = int(rng.randint(1, 501))
            skv = sq if rng.rand() < 0.5 else int(rng.randint(1, 501))
            while b * hq * sq * skv * dmax > WORK_LIMIT:
                sq, skv = max(1, sq // 2), max(1, skv // 2)
            kw.update(batch=b, sq=sq, skv=skv)
        out.append(kw)
    return out


CASES = _cases()


def _id(kw):
    shape = (f"thd{len(kw['seqlens'])}" if "seqlens" in kw else f"b{kw['batch']}_{kw['sq']}x{kw['skv']}")
    return f"{shape}-d{kw['d']}x{kw['dv']}-{kw['dtype']}-{kw['mask']}-w{kw['window_left']}-h{kw['hq']}_{kw['hkv']}"


@pytest.mark.parametrize("i", range(N_CASES), ids=[f"{i}-{_id(c)}" for i, c in enumerate(CASES)])
def test_fuzz(i):
    w = small(f"fuzz_{i}", **CASES[i])
    ok, msgs = run_and_check(w)
    assert ok, "\n".join(m for m in msgs if m.startswith("FAIL"))


WIDE = [i for i, c in enumerate(CASES) if max(c["d"], c["dv"]) > 256]


@pytest.mark.parametrize("i", WIDE, ids=[f"{i}-{_id(CASES[i])}" for i in WIDE])
def test_fuzz_stored_ds(i):
    """The same configurations with a head above 256 through the stored-dS backward (ATTN_FLAG_BWD_STORED_DS)."""
    w = small(f"fuzz_sds_{i}", **CASES[i])
    ok, msgs = run_and_check(w, stored_ds=True)
    assert ok, "\n".join(m for m in msgs if m.startswith("FAIL"))
