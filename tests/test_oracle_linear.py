"""Pins for oracle.linear_fwd_bwd: which tensor each scaling input reaches.

[AMAX] "Proposed method", bullet 2: every tensor's bias is
floor(log2(format max / amax)) less a configurable margin, so the margin
applies to X, W and dY alike. [FP8LM] "Proposed method", O1, Eq. 3: the
auto-scaling factor mu multiplies gradients only, so mu_log2 enters dY's
bias and neither X's nor W's.

Independent of the oracle's own steps: the biases come from the
exponent/mantissa closed form (math.frexp); the FP8 bytes from torch's
float8 conversion of the scaled float32 values (exact: bf16 times a power
of two), with elements whose scaled magnitude exceeds the format maximum
expected at the saturated code; the GEMM sums from torch's float8 decode
and a float64 product with each operand's own 2^-bias. A mu routed to X or
W, a margin applied to dY alone, or a dequantisation that forgets mu each
fail here."""
import math

import numpy as np
import pytest
import torch

from oracle import linear_fwd_bwd
from workloads import f32_to_bf16_bits

E4_MAX, E5_MAX = 448.0, 57344.0


def _closed_form_bias(bits, fmt_exp, margin, mu_log2):
    """floor(log2(1.75 * 2^E / amax)) - margin + mu_log2 from the fields of amax."""
    a = float(np.abs(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()).max())
    m, e = math.frexp(a)              # a = m 2^e, m in [0.5, 1)
    m, e = 2 * m, e - 1
    return fmt_exp - e - (1 if m > 1.75 else 0) - margin + mu_log2


def _bf16_f64(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double()


def _expected_codes(bits, bias, dtype, fmt_max, max_code):
    """torch's float8 cast of x * 2^bias where it stays in range; the
    saturated code (with the sign) where the scaled magnitude is above max."""
    v = torch.ldexp(_bf16_f64(bits), torch.tensor(float(bias), dtype=torch.float64))
    sat = v.abs() > fmt_max
    want = v.float().to(dtype).view(torch.uint8).numpy().copy()
    neg = (v < 0).numpy()
    want[sat.numpy()] = np.where(neg[sat.numpy()], 0x80 | max_code, max_code)
    return want, int(sat.sum())


def _decoded(codes, dtype, bias):
    return torch.from_numpy(codes).view(dtype).double() * 2.0 ** (-bias)


def _inputs(seed, M=48, K=80, N=64):
    g = np.random.Generator(np.random.PCG64(seed))
    X = f32_to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    W = f32_to_bf16_bits((0.02 * g.standard_normal((K, N))).astype(np.float32))
    dY = f32_to_bf16_bits((1e-5 * g.standard_normal((M, N))).astype(np.float32))
    return X, W, dY


@pytest.mark.parametrize("margin,mu_log2", [(1, 2), (1, 3), (2, -1), (-1, 0), (0, 1), (3, 0)])
def test_margin_on_all_tensors_mu_on_gradient_only(margin, mu_log2):
    X, W, dY = _inputs(100 + 10 * margin + mu_log2)
    out = linear_fwd_bwd(X, W, dY, margin=margin, mu_log2=mu_log2)
    bx = _closed_form_bias(X, 8, margin, 0)
    bw = _closed_form_bias(W, 8, margin, 0)
    bdy = _closed_form_bias(dY, 15, margin, mu_log2)
    assert (out["sx"]["bias"], out["sw"]["bias"], out["sdy"]["bias"]) == (bx, bw, bdy)
    for rec in (out["sx"], out["sw"], out["sdy"]):
        assert rec["scale"] == 2.0 ** rec["bias"] and rec["scale_inv"] == 2.0 ** -rec["bias"]

    # every FP8 byte, row-wise and transposed
    for key, bits, bias, dt, mx, mc in (("x8", X, bx, torch.float8_e4m3fn, E4_MAX, 0x7E),
                                        ("w8", W, bw, torch.float8_e4m3fn, E4_MAX, 0x7E),
                                        ("dy8", dY, bdy, torch.float8_e5m2, E5_MAX, 0x7B)):
        want, nsat = _expected_codes(bits, bias, dt, mx, mc)
        assert np.array_equal(out[key], want), key
        assert np.array_equal(out[key + "t"], want.T), key
        # a net shift margin - mu_log2 < 0 pushes the top of the range past max
        net = (margin - mu_log2) if key == "dy8" else margin
        assert (nsat > 0) == (net < 0), (key, nsat)

    # each GEMM undoes exactly its two operands' biases (mu included for dY)
    x = _decoded(out["x8"], torch.float8_e4m3fn, bx)
    w = _decoded(out["w8"], torch.float8_e4m3fn, bw)
    dy = _decoded(out["dy8"], torch.float8_e5m2, bdy)
    for key, ref in (("Y", x @ w), ("dX", dy @ w.T), ("dW", x.T @ dy)):
        c64 = out[key][1]
        assert np.allclose(c64, ref.numpy(), rtol=1e-12, atol=0), key


@pytest.mark.parametrize("margin,mu_log2", [(1, 1), (2, 2), (1, 0), (2, 0)])
def test_linear_with_margin_and_mu_approximates_real_product(margin, mu_log2):
    """With margin >= mu_log2 nothing saturates, so the three GEMMs stay
    within FP8 quantisation error of the real products whatever the margin
    and mu: a scale left on the output (mu not undone) is off by 2^mu."""
    X, W, dY = _inputs(7 + margin + 3 * mu_log2)
    out = linear_fwd_bwd(X, W, dY, margin=margin, mu_log2=mu_log2)
    x, w, dy = _bf16_f64(X).numpy(), _bf16_f64(W).numpy(), _bf16_f64(dY).numpy()
    # each margin step costs one bit of headroom; allow for it
    limit = 0.08 * 2 ** max(0, margin - 1)
    for key, ref in (("Y", x @ w), ("dX", dy @ w.T), ("dW", x.T @ dy)):
        rel = np.linalg.norm(out[key][1] - ref) / np.linalg.norm(ref)
        assert rel < limit, (key, rel)
