"""CPU checks of the floating-point acceptance rule (helpers.FpCheck /
check_fp) that every GPU parity test applies: accepted and rejected cases built
by hand, so that a mistake in the checker (a wrong window, a missing flip
count, a lost L2 term, a chunking error) fails here rather than letting a GPU
result through."""
import numpy as np
import pytest

import oracle as O
from helpers import ATOL, FLIP_WINDOW, FpCheck, check_fp

STEP4 = 2.0 ** -5          # bf16 spacing on [4, 8)


def bits(vals):
    return O.f64_to_bf16_rne(np.asarray(vals, dtype=np.float64))


def background(n=2000, seed=0):
    """Values whose float64 reference is exactly representable (no flips)."""
    rng = np.random.default_rng(seed)
    ref = O.bf16_bits_to_f64(bits(rng.standard_normal(n) * 6.0))
    return ref, bits(ref)


def test_exact_values_pass():
    ref, g = background()
    st = check_fp(g, ref, "exact")
    assert st["fail"] == 0 and st["flips"] == 0 and st["max_abs"] == 0.0
    assert st["big"] == int(np.count_nonzero(np.abs(ref) >= 4.0))
    assert st["rel_l2"] == 0.0


def test_a_flip_at_the_midpoint_is_accepted():
    ref, g = background()
    mid = 4.0 + STEP4 / 2                       # halfway between 4.0 and 4.03125
    assert O.bf16_bits_to_f64(bits([mid]))[0] == 4.0          # ties to even
    ref = np.append(ref, mid)
    g = np.append(g, bits([4.0 + STEP4]))       # the other side of the boundary
    st = check_fp(g, ref, "flip")
    assert st["flips"] == 1 and st["fail"] == 0
    assert st["max_abs"] == pytest.approx(STEP4)
    assert STEP4 > ATOL                         # a legitimate flip above 4 exceeds the bound


def test_a_flip_outside_the_window_fails():
    ref, g = background()
    r = 4.0 + STEP4 / 2 - 4 * FLIP_WINDOW * 4.0   # rounds to 4.0, far from the midpoint
    ref = np.append(ref, r)
    g = np.append(g, bits([4.0 + STEP4]))
    with pytest.raises(AssertionError, match="outside tolerance"):
        check_fp(g, ref, "far flip")


def test_two_steps_off_fails():
    ref, g = background()
    ref = np.append(ref, 4.0 + STEP4 / 2)
    g = np.append(g, bits([4.0 + 2 * STEP4]))   # not the neighbour
    with pytest.raises(AssertionError, match="outside tolerance"):
        check_fp(g, ref, "two steps")


def test_too_many_flips_fail():
    n = 400
    mids = 4.0 + STEP4 * (np.arange(n) % 64) + STEP4 / 2
    ref = mids.copy()
    g = bits(mids + STEP4 / 4)                  # every element on the other side
    with pytest.raises(AssertionError, match="too many boundary flips"):
        check_fp(g, ref, "systematic")


def test_relative_l2_bound():
    rng = np.random.default_rng(3)
    ref = rng.standard_normal(5000) * 0.25      # |x| < 2: a step and 1 % stay under the bound
    g = bits(ref * 1.01)                        # a 1 % scale error, within 2e-2 per element
    assert np.max(np.abs(O.bf16_bits_to_f64(g) - O.bf16_bits_to_f64(bits(ref)))) <= ATOL
    with pytest.raises(AssertionError, match="relative L2"):
        check_fp(g, ref, "scale")


def test_poison_fails():
    ref, g = background()
    g = g.copy()
    g[7] = O.POISON_BITS
    with pytest.raises(AssertionError, match="non-finite"):
        check_fp(g, ref, "poison")


def test_chunked_accumulation_equals_the_whole():
    rng = np.random.default_rng(5)
    ref = rng.standard_normal(3001) * 5.0
    g = bits(ref)
    flip_at = np.flatnonzero(np.abs(ref) >= 4.0)[:3]
    ref[flip_at] = O.bf16_bits_to_f64(g[flip_at]) + np.sign(ref[flip_at]) * STEP4 / 2
    g = bits(ref)
    g[flip_at] = bits(O.bf16_bits_to_f64(g[flip_at]) + np.sign(ref[flip_at]) * STEP4 * 1.01)
    whole = check_fp(g, ref, "whole")
    c = FpCheck("chunks")
    for lo in range(0, ref.size, 431):
        c.add(g[lo:lo + 431], ref[lo:lo + 431])
    parts = c.finish()
    for key in ("n", "fail", "flips", "big", "max_abs"):
        assert parts[key] == whole[key], key
    assert parts["rel_l2"] == pytest.approx(whole["rel_l2"], rel=1e-12)
