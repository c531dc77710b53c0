"""The float comparison itself (tests/parity.py): it must pass what a correct
kernel produces and fail what a plausible mistake produces, on the CPU."""

import numpy as np
import pytest

from tests import parity


def _case(seed=0, shape=(256, 256)):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape) * np.exp(rng.standard_normal(shape))


def test_one_rounding_passes():
    ref = _case()
    parity.check({"x": (parity.bf16_round(ref), ref)})


def test_fp32_accumulation_noise_passes():
    ref = _case(1)
    got = parity.bf16_round(ref * (1 + 2.0 ** -20 * np.random.default_rng(2).standard_normal(ref.shape)))
    parity.check({"x": (got, ref)})


def test_wrong_tile_fails():
    ref = _case(3)
    got = parity.bf16_round(ref)
    got[128:256, 0:128] = parity.bf16_round(ref[128:256, 0:128] * 1.01)
    with pytest.raises(AssertionError, match="local"):
        parity.check({"x": (got, ref)})


def test_wrong_row_fails():
    ref = _case(4)
    got = parity.bf16_round(ref)
    got[17] = parity.bf16_round(ref[17] * 1.004)
    with pytest.raises(AssertionError, match="local"):
        parity.check({"x": (got, ref)})


def test_truncation_fails():
    """Rounding toward zero instead of to nearest: every element off by up to
    one step, caught by the whole-tensor one-rounding bound."""
    ref = _case(5)
    u = np.asarray(ref, np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    got = u.view(np.float32).astype(np.float64)
    with pytest.raises(AssertionError, match="one-rounding"):
        parity.check({"x": (got, ref)})


def test_near_tie_flip_is_accepted_only_near_a_midpoint():
    ref = _case(6, (64, 64))
    one = parity.bf16_round(ref)
    step = parity._ulp_bf16(one)
    # a value just below the midpoint above its rounding: either neighbour is right
    ref[3, 3] = one[3, 3] + 0.5 * step[3, 3] * (1 - 2.0 ** -10)
    one = parity.bf16_round(ref)
    got = one.copy()
    got[3, 3] = one[3, 3] + parity._ulp_bf16(one[3, 3])
    assert parity.near_tie_ref(got, ref)[3, 3] == got[3, 3]
    # a one-step difference far from a midpoint is not excused
    got2 = one.copy()
    far = (np.abs(ref - (one + parity._ulp_bf16(one) / 2)) > 0.25 * parity._ulp_bf16(one)) & \
          (np.abs(ref - (one - parity._ulp_bf16(one) / 2)) > 0.25 * parity._ulp_bf16(one))
    i, j = np.argwhere(far)[0]
    got2[i, j] = one[i, j] + parity._ulp_bf16(one[i, j])
    assert parity.near_tie_ref(got2, ref)[i, j] == one[i, j]


def test_dominated_group_with_near_tie_flips_passes():
    """A group whose largest element holds much of its norm, with one-step
    flips of near-midpoint values (what bf16 hi + lo products in fp32 give)."""
    rng = np.random.default_rng(7)
    ref = rng.standard_normal((512, 64))
    ref[:4] *= 1e-2
    ref[0, 0] = 0.5
    one = parity.bf16_round(ref)
    step = parity._ulp_bf16(one)
    ref[0, 0] = one[0, 0] + 0.5 * step[0, 0] * (1 - 2.0 ** -12)
    one = parity.bf16_round(ref)
    got = one.copy()
    got[0, 0] = one[0, 0] + parity._ulp_bf16(one[0, 0])
    parity.check({"x": (got, ref)})
