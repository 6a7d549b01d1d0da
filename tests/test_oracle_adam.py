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
