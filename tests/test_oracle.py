"""The fp64 oracle against its pins (closed forms, invariants, brute force,
library routines and the FlashDecoding++ post's own equivalence check), and
the fp64 -> bf16 rounding used for the bf16-output tolerance."""
import math

import numpy as np
import pytest

import oracle
import workloads
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.default())


def test_split_merge_on_named_small_config():
    """The smallest named config (MHA, D=64, L=1024): split at several chunk sizes equals unsplit."""
    x = workloads.config_inputs(0)
    full = oracle.attention(x.q, x.k, x.v, x.seq_lens, x.scale)
    for chunk in (64, 100, 256, 1024):
        sp = oracle.split_attention(x.q, x.k, x.v, x.seq_lens, x.scale, chunk)
        assert np.max(np.abs(sp[0] - full[0])) < 1e-13
        assert np.max(np.abs(sp[1] - full[1])) < 1e-12


# ---------------------------------------------------------------------------
# fp64 -> bf16 rounding
# ---------------------------------------------------------------------------
def test_round_to_bf16_agrees_with_integer_rounding_on_fp32_values():
    """For values that are exact fp32, direct fp64 rounding equals the generator's
    independent integer-bit RNE rounding of fp32."""
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32),
                        (rng.standard_normal(1000) * 1e-30).astype(np.float32),
                        (rng.standard_normal(1000) * 1e30).astype(np.float32)])
    want = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(x)).astype(np.float64)
    got = oracle.round_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_round_to_bf16_ties_and_no_double_rounding():
    r = oracle.round_to_bf16
    assert r(1.0 + 2.0 ** -8) == 1.0                       # tie -> even (down)
    assert r(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6       # tie -> even (up)
    # Just above the tie: direct rounding goes up, while rounding through fp32
    # first would land on the tie and then go down to 1.0.
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7
    assert r(-(1.0 + 2.0 ** -8 + 2.0 ** -40)) == -(1.0 + 2.0 ** -7)
    assert r(2.0 ** -130) == 2.0 ** -130                   # subnormal, exact
    assert r(2.0 ** -134) == 0.0                           # half the smallest step -> even (0)
    assert r(3 * 2.0 ** -134) == 2.0 ** -132               # 1.5 steps -> 2 steps
    assert r(1e39) == math.inf and r(-1e39) == -math.inf
    assert r(0.0) == 0.0 and math.copysign(1.0, float(r(-0.0))) == -1.0
    assert np.isnan(r(np.nan))


def test_bf16_bits_of_rejects_unrepresentable():
    assert oracle.bf16_bits_of([1.0, -2.5])[0] == 0x3F80
    with pytest.raises(ValueError):
        oracle.bf16_bits_of([1.0 + 2.0 ** -10])
