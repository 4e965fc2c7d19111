"""CPU checks of the GPU comparison rules themselves (gpu_util): synthetic
"device" results built from the oracle with planted differences, each of
which the rules must accept when an upstream difference explains it and
reject when it does not."""

import numpy as np
import pytest

import oracle as O
from gpu_util import act_code_flips, check_elementwise

RNG = np.random.default_rng(99)


def _fp8_act_case(act, n=4000):
    gated = len(act) == 2
    h1 = O.bf16_round(RNG.standard_normal((8, (2 if gated else 1) * n)) * 1.3)
    a = O.activation(h1, act)
    codes, meta = O.quantize(a)
    return h1, a, codes, meta


@pytest.mark.parametrize("act", [("gelu",), ("silu", "linear")])
def test_act_codes_identical_pass(act):
    h1, a, codes, meta = _fp8_act_case(act)
    nd, n1, by_h1, ties = act_code_flips(codes, codes, h1, h1, a, meta["scale"], 1.0, act)
    assert nd == n1 == by_h1 == ties == 0


@pytest.mark.parametrize("act", [("gelu",), ("silu", "linear")])
def test_act_code_wrong_where_h1_agrees_fails(act):
    h1, a, codes, meta = _fp8_act_case(act)
    got = codes.copy()
    # a code one step up, at a value far from a tie: a quantiser error
    v = a * meta["scale"]
    mid_dist = np.abs(v - O.e4m3_decode(codes))
    i = np.unravel_index(np.argmin(np.where((np.abs(v) > 1.0) & (np.abs(v) < 200.0), mid_dist, np.inf)), v.shape)
    got[i] = got[i] + 1
    with pytest.raises(AssertionError):
        act_code_flips(got, codes, h1, h1, a, meta["scale"], 1.0, act)
    # a NaN code is never a rounding
    nan = codes.copy()
    nan[0, 0] = 0x7F
    with pytest.raises(AssertionError):
        act_code_flips(nan, codes, h1, h1, a, meta["scale"], 1.0, act)


def test_act_code_follows_h1_difference_passes():
    act = ("gelu",)
    h1, a, codes, meta = _fp8_act_case(act)
    # the "device" h1 one bf16 step up at a few places, codes from the moved values
    h_dev = h1.copy()
    sel = (np.arange(8), RNG.integers(0, h1.shape[1], 8))
    _, ex = np.frexp(np.abs(h1[sel]))
    h_dev[sel] = h1[sel] + np.sign(h1[sel]) * np.ldexp(1.0, ex - 8)
    dev_codes = O.e4m3_encode(O.activation(h_dev, act) * meta["scale"])
    nd, n1, by_h1, ties = act_code_flips(dev_codes, codes, h_dev, h1, a, meta["scale"], 1.0, act)
    assert ties == 0 and by_h1 == nd


def test_act_code_near_zero_many_steps_needs_h1_difference():
    act = ("gelu",)
    h1 = np.array([[1e-5, 2.0, -3.0, 0.5]])
    a = O.activation(h1, act)
    codes, meta = O.quantize(a)
    h_dev = np.array([[3e-5, 2.0, -3.0, 0.5]])
    dev_codes = O.e4m3_encode(O.activation(h_dev, act) * meta["scale"])
    assert O.e4m3_decode(dev_codes[0, 0]) != O.e4m3_decode(codes[0, 0])
    act_code_flips(dev_codes, codes, h_dev, h1, a, meta["scale"], 1.0, act)
    with pytest.raises(AssertionError):   # the same codes without the h1 difference
        act_code_flips(dev_codes, codes, h1, h1, a, meta["scale"], 1.0, act)


def test_elementwise_guard_catches_a_misplaced_chunk():
    ref = RNG.standard_normal((64, 256))
    got = O.bf16_round(ref * (1 + 1e-3 * RNG.standard_normal(ref.shape)))
    check_elementwise(got, ref, 2e-3, "clean")
    bad = got.copy()
    bad[5, 8:16] = bad[6, 8:16]          # one 16-byte chunk from the wrong row
    with pytest.raises(AssertionError):
        check_elementwise(bad, ref, 2e-3, "chunk")
