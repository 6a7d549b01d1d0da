"""Pins for oracle.scaling: amax, the exponent-bias rule, the cast.

Pinned against: hand-worked biases (tests/golden/bias_cases.txt); an
independent closed form from the binary exponent and mantissa of amax
(amax = m * 2^e, fmt_max = 1.75 * 2^E  =>  bias = E - e - [m > 1.75]),
exhaustively over every positive finite bf16 amax; float log2 away from
integer boundaries; scale equivariance; brute-force amax."""
import math

import numpy as np
import pytest

from oracle import (E4M3, E5M2, FLAG_CLAMPED, FLAG_NONFINITE, FLAG_ZERO, amax, bf16_to_f64,
                    cast, compute_bias, encode, f64_to_bf16_rne, fixed_record, saturated_count,
                    scale_record)
from tests import _golden
from workloads import f32_to_bf16_bits, random_bf16_bits

FMT = {"e4m3": E4M3, "e5m2": E5M2}
TOP_EXP = {"e4m3": 8, "e5m2": 15}   # fmt_max = 1.75 * 2^TOP_EXP


def test_bias_golden_cases():
    for name, a, margin, mu, bias in _golden.bias_cases():
        b, _ = compute_bias(a, FMT[name], margin, mu)
        assert b == bias, (name, a, margin, mu, b, bias)


def _frexp_rule(a, top):
    m, e = math.frexp(a)            # a = m * 2^e, m in [0.5, 1)
    m, e = 2 * m, e - 1             # m in [1, 2)
    return top - e - (1 if m > 1.75 else 0)


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_bias_exhaustive_all_bf16_amax(name):
    fmt, top = FMT[name], TOP_EXP[name]
    vals = bf16_to_f64(np.arange(0x0001, 0x7F80, dtype=np.uint16))
    for a in vals:
        b, flags = compute_bias(float(a), fmt)
        b_ref = _frexp_rule(float(a), top)
        b_ref_c = min(max(b_ref, -126), 126)
        assert b == b_ref_c, (a, b, b_ref)
        assert bool(flags & FLAG_CLAMPED) == (b_ref != b_ref_c)
        if b_ref == b_ref_c:
            # largest shift that keeps amax inside the format (exact in float64)
            assert a * 2.0 ** b <= fmt.max_finite < a * 2.0 ** (b + 1)


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_bias_float_log2_away_from_boundaries(name):
    fmt = FMT[name]
    g = np.random.Generator(np.random.PCG64(3))
    for a in np.exp2(g.uniform(-60, 60, size=2000)):
        r = math.log2(fmt.max_finite / a)
        if abs(r - round(r)) < 1e-9:
            continue
        b, _ = compute_bias(float(a), fmt)
        assert b == math.floor(r)


def test_bias_margin_mu_equivariance_and_clamp():
    for a in (1e-3, 0.37, 1.0, 5.5, 300.0):
        b0, _ = compute_bias(a, E4M3)
        assert compute_bias(a, E4M3, margin=1)[0] == b0 - 1
        assert compute_bias(a, E4M3, margin=3, mu_log2=2)[0] == b0 - 1
        assert compute_bias(2 * a, E4M3)[0] == b0 - 1        # doubling amax halves the scale
        assert compute_bias(a / 4, E4M3)[0] == b0 + 2
    b, f = compute_bias(2.0 ** -133, E4M3)
    assert (b, f) == (126, FLAG_CLAMPED)
    b, f = compute_bias(1.0, E5M2, mu_log2=200)
    assert (b, f) == (126, FLAG_CLAMPED)
    b, f = compute_bias(1.0, E4M3, margin=300)
    assert (b, f) == (-126, FLAG_CLAMPED)
    assert compute_bias(0.0, E4M3, margin=1, mu_log2=3) == (0, FLAG_ZERO)
    assert compute_bias(math.inf, E5M2) == (0, FLAG_NONFINITE)
    assert compute_bias(math.nan, E4M3) == (0, FLAG_NONFINITE)


def test_amax_brute_force_and_invariants():
    g = np.random.Generator(np.random.PCG64(11))
    bits = random_bf16_bits(5, (37, 53))
    ref = max(abs(float(v)) for v in bf16_to_f64(bits).reshape(-1))
    assert amax(bits) == ref
    perm = g.permutation(bits.reshape(-1))
    assert amax(perm) == ref
    assert amax(perm ^ np.uint16(0x8000)) == ref               # sign flips
    assert amax(np.zeros((4, 4), np.uint16)) == 0.0
    assert amax(np.full(3, 0x8000, np.uint16)) == 0.0           # -0
    assert amax(np.zeros(0, np.uint16)) == 0.0
    b = bits.copy().reshape(-1)
    b[17] = 0xFF80                                               # -inf
    assert amax(b) == math.inf
    b[3] = 0x7FC1                                                # NaN
    assert math.isnan(amax(b))


def test_scale_record_fields():
    x = f32_to_bf16_bits(np.array([[0.5, -3.0], [2.0, 1.0]], np.float32))
    r = scale_record(x, E4M3)
    assert r["amax"] == 3.0 and r["bias"] == 7 and r["flags"] == 0     # 448/3 = 149.3
    assert r["scale"] == 128.0 and r["scale_inv"] == 1 / 128.0
    r = scale_record(x, E5M2, margin=1, mu_log2=-1)
    assert r["bias"] == 14 - 1 - 1


def test_cast_definition_and_layouts():
    x = random_bf16_bits(9, (24, 40))
    for fmt, b in ((E4M3, 3), (E5M2, -5), (E4M3, 126)):
        q, qt = cast(x, fmt, b)
        assert q.shape == (24, 40) and qt.shape == (40, 24)
        assert np.array_equal(qt, q.T)
        ref = encode(bf16_to_f64(x) * 2.0 ** b, fmt)
        assert np.array_equal(q, ref)


def test_cast_scaling_direction_keeps_amax_in_range():
    """With the amax bias, the largest |x| lands in [max/2, max] of the
    format (no saturation at margin 0), and every scaled value is finite."""
    g = np.random.Generator(np.random.PCG64(5))
    for fmt in (E4M3, E5M2):
        for s in (1e-6, 0.02, 1.0, 37.0):
            x = f32_to_bf16_bits((g.standard_normal(4096) * s).astype(np.float32))
            r = scale_record(x, fmt)
            q, _ = cast(x, fmt, r["bias"])
            from oracle import decode_table
            dq = np.abs(decode_table(fmt)[q])
            assert fmt.max_finite / 2 <= dq.max() <= fmt.max_finite


def test_fixed_record_matches_amax_record_of_a_tensor_at_that_bias():
    """FP8-CSCALE: a fixed bias b gives the same scale and inverse as the
    amax rule on a tensor whose amax is fmt_max * 2^-b (where the rule lands
    exactly on b at margin 0), for every bias in range."""
    for fmt in (E4M3, E5M2):
        for b in range(-126, 127):
            a = fmt.max_finite * 2.0 ** -b
            if not (2.0 ** -133 <= a < 2.0 ** 128):
                continue
            bits = f64_to_bf16_rne(np.array([a, -a / 3]))
            if bf16_to_f64(bits)[0] != a:
                continue
            want = scale_record(bits, fmt)
            got = fixed_record(b)
            assert want["bias"] == b and want["flags"] == 0
            assert (got["bias"], got["scale"], got["scale_inv"], got["flags"]) == (
                b, want["scale"], want["scale_inv"], 0)
    for bad in (-127, 127):
        with pytest.raises(ValueError):
            fixed_record(bad)


@pytest.mark.parametrize("fmt,E", [(E4M3, 8), (E5M2, 15)])
def test_saturated_count_vs_bit_threshold_and_encoder(fmt, E):
    """The clipped-element count, exhaustively over every bf16 pattern and
    every bias: (1) it equals the count of magnitudes above the closed-form
    threshold pattern of max * 2^-bias (max = 1.75 * 2^E, so exponent field
    127 + E - bias and mantissa 0x60; no finite value above the bf16 range),
    NaN patterns excluded; (2) every counted element encodes to the +-max
    code."""
    allbits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    mag = allbits.astype(np.uint32) & 0x7FFF
    max_code = int(encode(np.array([fmt.max_finite]), fmt)[0])
    for b in range(-126, 127):
        e = 127 + E - b
        thr = (e << 7) | 0x60 if e <= 254 else 0x7F7F
        want = int(np.count_nonzero((mag > thr) & (mag <= 0x7F80)))
        assert saturated_count(allbits, fmt, b) == want, b
    for b in (-60, -1, 0, 1, 7, 30):
        x = bf16_to_f64(allbits)
        with np.errstate(invalid="ignore", over="ignore"):
            clipped = np.abs(np.ldexp(x, b)) > fmt.max_finite
        q = encode(np.ldexp(x[clipped], b), fmt)
        assert np.all((q & 0x7F) == max_code), b
