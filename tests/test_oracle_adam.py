"""Pins for oracle.adam (O2 optimizer state, test infrastructure only).

Pinned against: torch's float64 -> float16 conversion (the FP16 encoder);
the exponent/mantissa closed form of the bias rule for the FP16 maximum
65504, exhaustively over every positive finite bf16 amax; closed forms of
AdamW: at beta1 = beta2 = 0 and step 1 the update is lr * g / (|g| + eps);
with a constant gradient the bias-corrected moments are exact, so every
step moves w by the same amount; with g = 0 only the weight decay acts;
the update is odd in g. The FP8 encoder and the FP8 bias rule are pinned in
test_oracle_formats.py / test_oracle_scaling.py."""
import numpy as np
import pytest
import torch

from oracle import adam, bf16_to_f64, compute_bias, f64_to_bf16_rne


def test_fp16_encoder_matches_torch():
    g = np.random.Generator(np.random.PCG64(1))
    x = np.concatenate([
        g.standard_normal(20000) * 10.0 ** g.uniform(-9, 5, 20000),
        [0.0, -0.0, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 65504.0, 65519.99, 65520.0, 2.0 ** -24, 2.0 ** -25,
         3 * 2.0 ** -26, -2.0 ** -14, np.inf, -np.inf],
    ])
    want = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(adam.f64_to_f16_rne(x), want)
    # round trip of every finite FP16 pattern
    bits = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7C00) != 0x7C00
    assert np.array_equal(adam.f64_to_f16_rne(adam.f16_to_f64(bits[finite])), bits[finite])


def test_fp16_bias_rule_closed_form_all_bf16_amax():
    vals = bf16_to_f64(np.arange(1, 0x7F80, dtype=np.uint16))
    for a in vals:
        b, flags = compute_bias(float(a), adam.FP16_STORE)
        m, e = np.frexp(a)            # a = m * 2^e, m in [0.5, 1)
        m, e = 2 * m, e - 1           # m in [1, 2)
        want = 15 - e - (1 if m > 2 - 2.0 ** -10 else 0)
        clamped = min(max(want, -126), 126)
        assert (b, bool(flags)) == (clamped, clamped != want), a
        if clamped == want:
            assert a * 2.0 ** b <= 65504.0 < a * 2.0 ** (b + 1)


def test_adam_update_closed_forms():
    g = np.array([3e-5, -2e-3, 0.5, -1e-9])
    w = np.array([0.02, -0.01, 0.3, 1.0])
    z = np.zeros(4)
    lr, eps = 1e-3, 1e-8
    # beta = 0, step 1, no decay: a sign-like step of lr * g / (|g| + eps)
    _, _, wn = adam.adam_update(g, z, z, w, lr, 0.0, 0.0, eps, 0.0, 1)
    assert np.allclose(wn, w - lr * g / (np.abs(g) + eps), rtol=1e-15, atol=0)
    # constant gradient: bias correction makes every step equal
    m1, m2, wt = z, z, w.copy()
    for t in range(1, 8):
        m1, m2, wt = adam.adam_update(g, m1, m2, wt, lr, 0.9, 0.95, eps, 0.0, t)
        assert np.allclose(wt, w - t * lr * g / (np.abs(g) + eps), rtol=1e-12, atol=1e-15), t
    # no gradient: only the decoupled weight decay
    _, _, wn = adam.adam_update(z, z, z, w, lr, 0.9, 0.95, eps, 0.1, 3)
    assert np.array_equal(wn, w - lr * 0.1 * w)
    # odd in g (moments and update flip sign)
    a = adam.adam_update(g, 0.5 * g, g * g, w, lr, 0.9, 0.95, eps, 0.0, 4)
    b = adam.adam_update(-g, -0.5 * g, g * g, w, lr, 0.9, 0.95, eps, 0.0, 4)
    assert np.array_equal(a[0], -b[0]) and np.array_equal(a[1], b[1])
    assert np.allclose(a[2] - w, -(b[2] - w), rtol=1e-12, atol=0)   # (w - d) - w cancels


def test_master_init_exact_in_fp16_normal_range():
    g = np.random.Generator(np.random.PCG64(2))
    wb = f64_to_bf16_rne(g.standard_normal(4096) * 0.02)
    r = adam.master_init(wb)
    w = bf16_to_f64(wb)
    back = adam.f16_to_f64(r["w16"]) * r["rec"]["scale_inv"]
    normal = np.abs(w) * r["rec"]["scale"] >= 2.0 ** -14
    assert np.array_equal(back[normal], w[normal])
    assert np.abs(w).max() * r["rec"]["scale"] <= 65504.0


# ---- adam_step as a whole: a scalar re-derivation, independent of the
# oracle's tables, encoders and bias rule ----------------------------------
import math
import struct


def _dec_fields(code, exp_bits, man_bits, exp_bias):
    """Finite FP8 value from the sign / exponent / mantissa fields."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> man_bits) & ((1 << exp_bits) - 1)
    m = code & ((1 << man_bits) - 1)
    if e == 0:
        return s * m * 2.0 ** (1 - exp_bias - man_bits)
    return s * (1 + m / (1 << man_bits)) * 2.0 ** (e - exp_bias)


def _dec_e5m2(c):
    return _dec_fields(c, 5, 2, 15)


def _dec_e4m3(c):
    return _dec_fields(c, 4, 3, 7)


def _f16_dec(bits):
    return struct.unpack("<e", struct.pack("<H", int(bits)))[0]


def _f16_enc(x):
    # CPython's binary16 packing rounds to nearest, ties to even
    return struct.unpack("<H", struct.pack("<e", x))[0]


_E4_FINITE = [(c, _dec_e4m3(c)) for c in range(0x7F)]      # codes 0x00..0x7E, values 0 .. 448


def _e4m3_nearest(x):
    """E4M3 code by brute-force nearest search (ties to the even code); the
    magnitude is at most 448 here."""
    a = abs(x)
    best = min(_E4_FINITE, key=lambda cv: (abs(cv[1] - a), cv[0] & 1))
    return best[0] | (0x80 if math.copysign(1.0, x) < 0 else 0)


def _bias_closed(amax, exp_max, top_mant):
    """floor(log2(max / amax)) for max = top_mant * 2^exp_max, from frexp."""
    m, e = math.frexp(amax)
    m, e = 2 * m, e - 1
    return exp_max - e - (1 if m > top_mant else 0)


def _bf16_rne(v):
    """bf16 bits of v, one rounding to nearest even (8 significant bits)."""
    if v == 0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    a = abs(v)
    _, e = math.frexp(a)
    q = 2.0 ** (max(e - 1, -126) - 7)
    r = round(a / q) * q                      # Python round: half to even, a / q exact
    bits = struct.unpack("<I", struct.pack("<f", r))[0] >> 16
    return bits | (0x8000 if v < 0 else 0)


def _scalar_adamw(g, m1, m2, w, lr, b1, b2, eps, wd, t):
    m1 = b1 * m1 + (1 - b1) * g
    m2 = b2 * m2 + (1 - b2) * g * g
    step = (m1 / (1 - b1 ** t)) / (math.sqrt(m2 / (1 - b2 ** t)) + eps) + wd * w
    return m1, m2, w - lr * step


def _stored_state(seed, n=16):
    """Random stored tensors: E5M2 gradient codes, E4M3 m1 codes, FP16 m2 and
    master bits, each with a power-of-two scale_inv far from 1 (so that a
    scale / scale_inv swap or a dropped scale is visible)."""
    g = np.random.Generator(np.random.PCG64(seed))
    gc = [int(c) for c in g.integers(0, 0x7B, n)]            # finite E5M2, up to 0x7A
    gc = [c | (0x80 if s else 0) for c, s in zip(gc, g.integers(0, 2, n))]
    m1c = [int(c) | (0x80 if s else 0) for c, s in zip(g.integers(0, 0x7E, n), g.integers(0, 2, n))]
    m2b = [int(b) for b in g.integers(0x0400, 0x7800, n)]     # positive normal FP16
    wb = [int(b) | (0x8000 if s else 0) for b, s in zip(g.integers(0x2000, 0x7800, n), g.integers(0, 2, n))]
    return gc, m1c, m2b, wb


@pytest.mark.parametrize("seed", [1, 2, 3])
@pytest.mark.parametrize("hp", [(1e-3, 0.9, 0.95, 1e-8, 0.1, 3), (3e-4, 0.8, 0.999, 1e-6, 0.0, 1),
                                (1e-2, 0.0, 0.0, 1e-8, 0.0, 1)])
def test_adam_step_matches_hand_written_scalar_adamw(seed, hp):
    lr, b1, b2, eps, wd, t = hp
    gc, m1c, m2b, wb = _stored_state(seed)
    sg, s1, s2, sw = 2.0 ** -20, 2.0 ** -9, 2.0 ** -30, 2.0 ** -13      # scale_inv of each record
    got = adam.adam_step(np.array(gc, np.uint8), sg, np.array(m1c, np.uint8), s1, np.array(m2b, np.uint16), s2,
                         np.array(wb, np.uint16), sw, lr, b1, b2, eps, wd, t)
    new = [_scalar_adamw(_dec_e5m2(a) * sg, _dec_e4m3(b) * s1, _f16_dec(c) * s2, _f16_dec(d) * sw,
                         lr, b1, b2, eps, wd, t) for a, b, c, d in zip(gc, m1c, m2b, wb)]
    m1n = np.array([v[0] for v in new])
    m2n = np.array([v[1] for v in new])
    wn = np.array([v[2] for v in new])
    assert np.allclose(got["m1"], m1n, rtol=1e-14, atol=0)
    assert np.allclose(got["m2"], m2n, rtol=1e-14, atol=0)
    assert np.allclose(got["w"], wn, rtol=1e-14, atol=0)
    # new records: just in time, from the NEW tensors' max |value|
    b1n = _bias_closed(float(np.abs(m1n).max()), 8, 1.75)
    b2n = _bias_closed(float(np.abs(m2n).max()), 15, 2 - 2.0 ** -10)
    bwn = _bias_closed(float(np.abs(wn).max()), 15, 2 - 2.0 ** -10)
    assert (got["m1_rec"]["bias"], got["m2_rec"]["bias"], got["w_rec"]["bias"]) == (b1n, b2n, bwn)
    for rec in (got["m1_rec"], got["m2_rec"], got["w_rec"]):
        assert rec["scale"] == 2.0 ** rec["bias"] and rec["scale_inv"] == 2.0 ** -rec["bias"]
    # re-encoded with the new scales (multiply by 2^bias before the cast)
    assert [int(c) for c in got["m1_codes"]] == [_e4m3_nearest(math.ldexp(v, b1n)) for v in got["m1"]]
    assert [int(c) for c in got["m2_bits"]] == [_f16_enc(math.ldexp(v, b2n)) for v in got["m2"]]
    assert [int(c) for c in got["w16"]] == [_f16_enc(math.ldexp(v, bwn)) for v in got["w"]]
    assert [int(c) for c in got["w_bf16"]] == [_bf16_rne(v) for v in got["w"]]


def test_adam_step_records_follow_the_new_tensor():
    """Records are taken from the updated tensors, not kept from the old
    ones: a large learning rate moves w far enough that its bias changes."""
    gc, m1c, m2b, wb = _stored_state(4)
    sw = 2.0 ** -13
    w_old = max(abs(_f16_dec(b) * sw) for b in wb)
    got = adam.adam_step(np.array(gc, np.uint8), 2.0 ** -20, np.array(m1c, np.uint8), 2.0 ** -9,
                         np.array(m2b, np.uint16), 2.0 ** -30, np.array(wb, np.uint16), sw,
                         8.0, 0.9, 0.95, 1e-8, 0.0, 1)
    assert _bias_closed(w_old, 15, 2 - 2.0 ** -10) != got["w_rec"]["bias"]
    assert got["w_rec"]["bias"] == _bias_closed(float(np.abs(got["w"]).max()), 15, 2 - 2.0 ** -10)


def test_adam_step_sign_step_and_zero_gradient_closed_forms():
    gc, m1c, m2b, wb = _stored_state(5)
    sg, s1, s2, sw = 2.0 ** -20, 2.0 ** -9, 2.0 ** -30, 2.0 ** -13
    g = np.array([_dec_e5m2(c) * sg for c in gc])
    w = np.array([_f16_dec(b) * sw for b in wb])
    # beta1 = beta2 = 0, step 1, no decay: w - lr g / (|g| + eps), whatever the moments held
    got = adam.adam_step(np.array(gc, np.uint8), sg, np.array(m1c, np.uint8), s1, np.array(m2b, np.uint16), s2,
                         np.array(wb, np.uint16), sw, 1e-3, 0.0, 0.0, 1e-8, 0.0, 1)
    assert np.allclose(got["w"], w - 1e-3 * g / (np.abs(g) + 1e-8), rtol=1e-13, atol=0)
    assert np.allclose(got["m1"], g, rtol=1e-15, atol=0) and np.allclose(got["m2"], g * g, rtol=1e-15, atol=0)
    # zero gradient (all codes 0): the moments decay by beta, and the weight
    # moves by lr * (m1_hat / (sqrt(m2_hat) + eps) + wd * w) of the decayed moments
    z = np.zeros(len(gc), np.uint8)
    m1 = np.array([_dec_e4m3(c) * s1 for c in m1c])
    m2 = np.array([_f16_dec(b) * s2 for b in m2b])
    got = adam.adam_step(z, sg, np.array(m1c, np.uint8), s1, np.array(m2b, np.uint16), s2,
                         np.array(wb, np.uint16), sw, 1e-3, 0.9, 0.95, 1e-8, 0.1, 2)
    assert np.allclose(got["m1"], 0.9 * m1, rtol=1e-15, atol=0)
    assert np.allclose(got["m2"], 0.95 * m2, rtol=1e-15, atol=0)
    mh, vh = 0.9 * m1 / (1 - 0.81), 0.95 * m2 / (1 - 0.9025)
    assert np.allclose(got["w"], w - 1e-3 * (mh / (np.sqrt(vh) + 1e-8) + 0.1 * w), rtol=1e-13, atol=0)


def test_adam_step_stored_values_round_trip():
    """What adam_step stores decodes (times the new scale_inv) to the new
    values within half a unit of the storage format at that scale."""
    gc, m1c, m2b, wb = _stored_state(6, n=64)
    got = adam.adam_step(np.array(gc, np.uint8), 2.0 ** -20, np.array(m1c, np.uint8), 2.0 ** -9,
                         np.array(m2b, np.uint16), 2.0 ** -30, np.array(wb, np.uint16), 2.0 ** -13,
                         1e-3, 0.9, 0.95, 1e-8, 0.01, 2)
    for vals, stored, dec, mbits, emin, rec in (
            (got["m1"], got["m1_codes"], _dec_e4m3, 3, -6, got["m1_rec"]),
            (got["m2"], got["m2_bits"], _f16_dec, 10, -14, got["m2_rec"]),
            (got["w"], got["w16"], _f16_dec, 10, -14, got["w_rec"])):
        for v, c in zip(vals, stored):
            s = math.ldexp(v, rec["bias"])
            back = dec(int(c))
            _, e = math.frexp(abs(s)) if s else (0, emin + 1)
            unit = 2.0 ** (max(e - 1, emin) - mbits)
            assert abs(back - s) <= unit / 2, (v, c)
