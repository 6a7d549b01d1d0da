"""Pins for oracle.formats / oracle.bf16: decode table, encoder, bf16 rounding.

Pinned against: hand-worked code values (tests/golden), torch's CPU float8
conversions (a library routine) in the range where they saturate the same
way, and an independent brute-force nearest-value encoder, exhaustively over
every bf16 pattern times every exponent bias."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import E4M3, E5M2, decode_table, encode, bf16_to_f64, f64_to_bf16_rne, bf16_ulp
from tests import _golden

FMT = {"e4m3": E4M3, "e5m2": E5M2}
TORCH_DT = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_decode_matches_torch_all_codes(name):
    t = decode_table(FMT[name])
    ref = torch.arange(256, dtype=torch.uint8).view(TORCH_DT[name]).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(t), np.isnan(ref))
    ok = ~np.isnan(t)
    assert np.array_equal(t[ok], ref[ok])
    assert np.array_equal(np.signbit(t[ok]), np.signbit(ref[ok]))


def test_decode_golden_values():
    for name, code, val in _golden.fp8_values():
        got = decode_table(FMT[name])[code]
        if math.isnan(val):
            assert math.isnan(got), (name, hex(code))
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), (name, hex(code), got, val)


def test_code_class_counts_and_extremes():
    t4, t5 = decode_table(E4M3), decode_table(E5M2)
    assert np.isfinite(t4).sum() == 254 and np.isnan(t4).sum() == 2 and np.isinf(t4).sum() == 0
    assert np.isfinite(t5).sum() == 248 and np.isnan(t5).sum() == 6 and np.isinf(t5).sum() == 2
    assert np.nanmax(t4) == 448.0 == E4M3.max_finite
    assert np.nanmax(t5[np.isfinite(t5)]) == 57344.0 == E5M2.max_finite
    assert t4[E4M3.max_code] == 448.0 and t5[E5M2.max_code] == 57344.0
    # finite values are symmetric in sign
    for t in (t4, t5):
        fin = np.isfinite(t[:128])
        assert np.array_equal(t[:128][fin], -t[128:][fin])


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_round_trip_finite_codes(name):
    fmt = FMT[name]
    t = decode_table(fmt)
    codes = np.array([c for c in range(256) if np.isfinite(t[c])], dtype=np.uint8)
    assert np.array_equal(encode(t[codes], fmt), codes)


def test_encode_golden_cases():
    for name, x, code in _golden.encode_cases():
        got = int(encode(np.array([x]), FMT[name])[0])
        assert got == code, (name, x, hex(got), hex(code))


def _nearest_encode(values, fmt):
    """Independent encoder: nearest finite FP8 value by a search over the
    sorted table (no binade arithmetic); ties go to the code with an even
    last bit; nothing lies beyond the largest finite value, so magnitudes
    above it land on it (saturation). Sign taken from the input."""
    t = decode_table(fmt)
    pos_codes = np.array([c for c in range(128) if np.isfinite(t[c])], dtype=np.int64)
    pos_vals = t[pos_codes]
    order = np.argsort(pos_vals, kind="stable")
    pos_vals, pos_codes = pos_vals[order], pos_codes[order]
    v = np.asarray(values, dtype=np.float64)
    a = np.abs(v)
    # anything at or beyond the largest finite value has that value as its
    # nearest finite neighbour (clamping first avoids float64 cancellation)
    a = np.minimum(np.where(np.isnan(a), 0.0, a), pos_vals.max())
    hi = np.clip(np.searchsorted(pos_vals, a, side="left"), 0, len(pos_vals) - 1)
    lo = np.clip(hi - 1, 0, len(pos_vals) - 1)
    dlo = np.abs(a - pos_vals[lo])
    dhi = np.abs(pos_vals[hi] - a)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((pos_codes[hi] & 1) == 0))
    code = np.where(pick_hi, pos_codes[hi], pos_codes[lo]).astype(np.uint8)
    code |= (np.signbit(v).astype(np.uint8) << 7)
    code = np.where(np.isnan(v), 0x7F | (np.signbit(v).astype(np.uint8) << 7), code)
    return code.astype(np.uint8)


ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_encode_exhaustive_vs_nearest_search(name):
    """Every bf16 pattern (NaN and inf included) times every bias in
    [-126, 126]: the arithmetic encoder equals the brute-force search."""
    fmt = FMT[name]
    x = bf16_to_f64(ALL_BF16)
    for b0 in range(-126, 127, 23):
        bs = np.arange(b0, min(b0 + 23, 127))
        v = np.ldexp(x[None, :], bs[:, None]).reshape(-1)
        got = encode(v, fmt)
        ref = _nearest_encode(v, fmt)
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, (name, v[bad[:5]], got[bad[:5]], ref[bad[:5]])


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_encode_matches_torch_below_overflow(name):
    """torch's float32 -> float8 conversion (round to nearest even) agrees
    wherever it cannot overflow; above that torch yields NaN/inf while the
    oracle saturates (a reading)."""
    fmt = FMT[name]
    limit = 464.0 if name == "e4m3" else 61440.0
    x = bf16_to_f64(ALL_BF16)
    for b in (-8, 0, 5, 9, 17, 29, 40):
        v = np.ldexp(x, b)
        keep = np.isfinite(v) & (np.abs(v) < limit) & (np.abs(v) > 2.0 ** -140)
        v = v[keep]
        ref = torch.from_numpy(v.astype(np.float32)).to(TORCH_DT[name]).view(torch.uint8).numpy()
        assert np.array_equal(encode(v, fmt), ref), (name, b)


def test_bf16_rne_against_torch_float32_inputs():
    """float32-exact inputs: torch's float32 -> bf16 rounding is a single
    round-to-nearest-even, so the two must agree bit for bit."""
    g = np.random.Generator(np.random.PCG64(7))
    u = g.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # include exact halfway cases
    u[:1000] = (u[:1000] & 0xFFFF0000) | 0x8000
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = f64_to_bf16_rne(f.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_rne_double_rounding_case():
    """A float64 just above a bf16 halfway point must round up: a naive
    float64 -> float32 -> bf16 path would round it down (ties-to-even)."""
    v = 1.0 + 2.0 ** -8 + 2.0 ** -40           # halfway 1 .. 1+2^-7, plus a bit
    assert int(f64_to_bf16_rne(np.array([v]))[0]) == 0x3F81
    assert int(f64_to_bf16_rne(np.array([1.0 + 2.0 ** -8]))[0]) == 0x3F80   # exact tie -> even
    assert int(f64_to_bf16_rne(np.array([-(1.0 + 3 * 2.0 ** -8)]))[0]) == 0xBF82
    big = (2.0 - 2.0 ** -8) * 2.0 ** 127
    assert int(f64_to_bf16_rne(np.array([big]))[0]) == 0x7F80                 # rounds to inf
    assert int(f64_to_bf16_rne(np.array([np.nextafter(big, 0)]))[0]) == 0x7F7F


def test_bf16_widen_and_ulp():
    assert bf16_to_f64(np.array([0x3F80], dtype=np.uint16))[0] == 1.0
    assert bf16_to_f64(np.array([0x0001], dtype=np.uint16))[0] == 2.0 ** -133
    assert bf16_ulp(np.array([1.0, 1.99, 2.0, -3.0, 0.0, 2.0 ** -130])).tolist() == [
        2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -6, 2.0 ** -133, 2.0 ** -133]
    # ulp equals the gap to the next bf16 value, for every positive normal pattern
    bits = np.arange(0x0080, 0x7F7F, dtype=np.uint16)
    gap = bf16_to_f64(bits + 1) - bf16_to_f64(bits)
    assert np.array_equal(bf16_ulp(bf16_to_f64(bits)), gap)
