"""CPU: the fixed-bound arithmetic of the parity tests (parity_util.fixed_bound).

The spacing of bf16 values is 2^-7 in [1, 2) and 2^-4 in [8, 16); of fp16 values 2^-10
in [1, 2). Below |ref| = 4 (bf16) / 8 (fp16) the bound is the literal 2e-2 / 5e-3; above,
one spacing of the dtype; LSE keeps 1e-3 absolute everywhere. Also checked against the
dtypes themselves: the next representable value after x lies ulp(x) above it.
"""

import numpy as np
import torch

from parity_util import BOUND, compare, fixed_bound, ulp


def test_spacings():
    assert ulp(np.array([1.0, 1.5, 8.8, 0.75]), "bf16").tolist() == [2 ** -7, 2 ** -7, 2 ** -4, 2 ** -8]
    assert ulp(np.array([1.0, 3.0, 9.0]), "fp16").tolist() == [2 ** -10, 2 ** -9, 2 ** -7]


def test_spacing_is_the_gap_to_the_next_stored_value():
    rng = np.random.default_rng(0)
    for name, dt in (("bf16", torch.bfloat16), ("fp16", torch.float16)):
        x = torch.from_numpy(rng.uniform(0.01, 60.0, 2000)).to(dt)
        gap = (torch.nextafter(x, torch.full_like(x, np.inf)).double() - x.double()).numpy()
        assert np.allclose(gap, ulp(x.double().numpy(), name)), name


def test_bounds_literal_below_the_crossover_and_one_spacing_above():
    ref = np.array([0.0, 0.5, 3.99, 4.0, 8.8, -8.8, 100.0])
    b = fixed_bound(ref, "bf16")
    assert (b[:3] == BOUND["bf16"]).all()
    assert b[3] == 2 ** -5 and b[4] == 2 ** -4 and b[5] == 2 ** -4 and b[6] == 2 ** 6 / 128
    f = fixed_bound(np.array([7.9, 8.0, 20.0]), "fp16")
    assert f[0] == BOUND["fp16"] and f[1] == 2 ** -7 and f[2] == 2 ** -6
    assert (fixed_bound(np.array([1.0, 50.0]), "bf16", is_lse=True) == 1e-3).all()


def test_compare_fixed_bound_and_floor_rules():
    ref = np.array([1.1, 0.5, -9.0])
    bump = np.array([0.0205, 0.0, 0.0])
    # over the literal bound where the floor is over it too and no more accurate: passes (1 x floor)
    assert compare("t", ref + bump, ref, ref + bump, "bf16")[0]
    # the same error where the floor meets the bound: fails
    assert not compare("t", ref + bump, ref, ref + np.array([0.019, 0, 0]), "bf16")[0]
    # under the bound but more than twice the floor's error: fails
    assert not compare("t", ref + np.array([0.01, 0, 0]), ref, ref + np.array([0.004, 0, 0]), "bf16")[0]
    # one bf16 spacing (1/16) allowed at |ref| = 9, not more
    assert compare("t", ref + np.array([0, 0, 0.06]), ref, ref + np.array([0, 0, 0.05]), "bf16")[0]
    assert not compare("t", ref + np.array([0, 0, 0.07]), ref, ref + np.array([0, 0, 0.05]), "bf16")[0]
    # unwritten (NaN) elements fail
    assert not compare("t", np.array([np.nan, 0.5, -9.0]), ref, ref, "bf16")[0]
    # LSE: -inf rows must match exactly, others within 1e-3
    lref = np.array([-np.inf, 2.0])
    assert compare("l", np.array([-np.inf, 2.0005]), lref, np.array([-np.inf, 2.0004]), "bf16", is_lse=True)[0]
    assert not compare("l", np.array([0.0, 2.0]), lref, lref, "bf16", is_lse=True)[0]
