"""Property checks of the oracle's activation quantizers over generated blocks
(hypothesis), beside the fixed pins in test_oracle_pins.py.  Each property follows
from the definition the pages give (codeloopback Examples 2-4; candle BlockQ8_0 /
BlockQ8K) without restating its arithmetic:
  - symmetry: quantizing -x gives the same scale and negated codes (amax is
    symmetric, halves round away from zero);
  - fixed point: quantizing the dequantized values gives the same bytes
    (codeloopback Example 4) whenever the stored scale is a finite nonzero number
    (for Q8_0 that includes f16 subnormal scales);
  - power-of-two scaling: x * 2^k gives the same codes and a scale times 2^k while
    the scale stays a normal number of its storage format;
  - Q8_K bsums are the sums of their 16 codes, codes lie in [-127, 127] and the
    largest magnitude maps to +-127;
  - Q8_1 (the reading of the _1 types' activation block) carries Q8_0's bytes for d
    and the codes, its sum field changes sign with x, and it lies within its two
    f16 roundings of the sum of the codes times the stored d.
Blocks whose largest magnitude is below 127 * 2^-128 are left out of the
symmetry, fixed-point and range properties: there 1 / d overflows to infinity and the codes
saturate to the int8 range, -128 included (the reading the C ABI documents).
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import oracle as o

SETTINGS = settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
ID_FINITE = 127 * 2.0 ** -128 * 1.01  # smallest amax whose 1 / (amax / 127) stays finite


def finite_id(x):
    return float(np.max(np.abs(x))) >= ID_FINITE


def blocks(n):
    """n float32 values: a magnitude scale (tiny to huge) times values that mix
    zeros, halves, +-1 and uniform draws (from a drawn seed: generating long lists
    element by element would be slow)."""
    def make(t):
        scale, seed = t
        rng = np.random.default_rng(seed)
        v = rng.uniform(-1.0, 1.0, n).astype(np.float32)
        special = rng.random(n) < 0.3
        v[special] = rng.choice(np.array([0.0, 0.5, -0.5, 1.0, -1.0], dtype=np.float32), int(special.sum()))
        return (np.float32(scale) * v).astype(np.float32)
    return st.tuples(st.sampled_from([1e-40, 1e-30, 1e-8, 1e-3, 1.0, 7.5, 1e4, 1e30, 3e37]),
                     st.integers(0, 2 ** 32 - 1)).map(make)


def split(t, b):
    """(scale as f32, int8 codes) of one quantized block."""
    if t == o.Q8_0:
        d = np.frombuffer(b[:2].tobytes(), np.float16)[0].astype(np.float32)
        return d, b[2:34].view(np.int8)
    d = np.frombuffer(b[:4].tobytes(), np.float32)[0]
    return d, b[4:260].view(np.int8)


@pytest.mark.parametrize("t,n", [(o.Q8_0, 32), (o.Q8_K, 256)])
@SETTINGS
@given(data=st.data())
def test_sign_symmetry(t, n, data):
    x = data.draw(blocks(n))
    if not finite_id(x):
        return
    d1, c1 = split(t, o.quantize(t, x))
    d2, c2 = split(t, o.quantize(t, -x))
    assert d1 == d2
    assert np.array_equal(c2.astype(np.int32), -c1.astype(np.int32))


@pytest.mark.parametrize("t,n", [(o.Q8_0, 32), (o.Q8_K, 256), (o.Q4_0, 32)])
@SETTINGS
@given(data=st.data())
def test_requantizing_dequantized_values_is_a_fixed_point(t, n, data):
    x = data.draw(blocks(n))
    b = o.quantize(t, x)
    y = o.dequantize(t, b, n) if t != o.Q8_K else _dequant_q8_K(b)
    d = np.frombuffer(b[:2].tobytes(), np.float16)[0] if t != o.Q8_K else split(t, b)[0]
    if not finite_id(x) or not np.all(np.isfinite(y)) or d == 0:
        return  # saturated codes, or a scale that overflowed or underflowed its format
    assert np.array_equal(o.quantize(t, y), b)


def _dequant_q8_K(b):
    d, c = split(o.Q8_K, b)
    return (c.astype(np.float32) * d).astype(np.float32)


@pytest.mark.parametrize("t,n,k", [(o.Q8_0, 32, 3), (o.Q8_0, 32, -5), (o.Q8_K, 256, 7), (o.Q8_K, 256, -9)])
@SETTINGS
@given(data=st.data())
def test_power_of_two_scaling(t, n, k, data):
    x = data.draw(blocks(n))
    with np.errstate(over="ignore"):
        xs = (x * np.float32(2.0 ** k)).astype(np.float32)
    if not np.all(np.isfinite(xs)):
        return  # the scaled inputs themselves overflow f32
    d1, c1 = split(t, o.quantize(t, x))
    d2, c2 = split(t, o.quantize(t, xs))
    amax = float(np.max(np.abs(x)))
    lo, hi = (6.2e-5, 6.0e4) if t == o.Q8_0 else (1.2e-38, 3.0e38)  # normal range of the scale
    if not (lo * 4 < amax / 127 < hi / 4 and lo * 4 < amax / 127 * 2.0 ** k < hi / 4):
        return
    if np.any((x != 0) & (np.abs(x) < 1e-37)) or np.any(np.abs(x * 2.0 ** k)[x != 0] < 1e-37):
        return  # subnormal inputs lose bits when scaled
    assert np.array_equal(c1, c2)
    assert d2 == np.float32(d1 * np.float32(2.0 ** k))


@SETTINGS
@given(x=blocks(256))
def test_q8_K_bsums_range_and_extreme(x):
    b = o.quantize(o.Q8_K, x)
    d, c = split(o.Q8_K, b)
    bs = b[260:292].view(np.int16)
    assert np.array_equal(bs.astype(np.int64), c.astype(np.int64).reshape(16, 16).sum(axis=1))
    if not finite_id(x):
        return
    assert np.all(np.abs(c.astype(np.int32)) <= 127)
    if d > 0 and np.isfinite(d):
        i = int(np.argmax(np.abs(x)))
        assert abs(int(c[i])) == 127


@SETTINGS
@given(x=blocks(32))
def test_q8_1_d_and_codes_are_q8_0s(x):
    b1 = o.quantize(o.Q8_1, x)
    b0 = o.quantize(o.Q8_0, x)
    assert b1[0:2].tobytes() == b0[0:2].tobytes() and b1[4:36].tobytes() == b0[2:34].tobytes()


@SETTINGS
@given(x=blocks(32))
def test_q8_1_sum_field_sign_and_bound(x):
    if not finite_id(x):
        return
    b = o.quantize(o.Q8_1, x)
    s = np.frombuffer(b[2:4].tobytes(), np.float16)[0]
    s_neg = np.frombuffer(o.quantize(o.Q8_1, -x)[2:4].tobytes(), np.float16)[0]
    d16 = np.float64(np.frombuffer(b[0:2].tobytes(), np.float16)[0])
    S = int(b[4:36].view(np.int8).astype(np.int64).sum())
    if not np.isfinite(s) or not np.isfinite(d16):
        return
    assert s_neg == -s and (S != 0 or s == 0)
    # s rounds S * d32 (d32 the unrounded scale, d16 its f16 rounding) twice: to f32,
    # then to f16; d16 is within 2^-11 of d32 (or 2^-25 below the f16 normal range)
    s = np.float64(s)
    bound = abs(S) * (2.0 ** -10 * d16 + 2.0 ** -24) + 2.0 ** -11 * abs(s) + 2.0 ** -24
    assert abs(s - S * d16) <= bound, (s, S, d16)
