"""O2 precision-decoupled Adam step (fp8_adam_init_master, fp8_adam_step,
fp8_adam_step_spec) through the C ABI, against oracle.adam.

[FP8-LM reading note, "Proposed method", O2: first moment FP8, second
moment FP16, master weights FP16 with tensor scaling.] Each step starts
from the kernel's own stored state (codes, FP16 bits and records), so errors
do not accumulate across steps. The kernel updates in fp32, the oracle in
float64, so a stored value may land on the neighbouring code where the two
straddle a rounding midpoint: every stored value must be within one unit
of the storage format (at the record's scale) of the oracle's, plus 2e-6
of the magnitudes the fp32 arithmetic combines (|w| + |w' - w| for the
weights, |beta1 m1| + |(1 - beta1) g| for the first moment: where the
update nearly cancels w, the fp32 error is relative to the operands, not
to the small result); the new per-tensor biases must equal the oracle's unless the
oracle's max lies within 1e-5 (relative) of a power-of-two boundary.
Master-weight initialisation is bit-exact. The one-pass step
(fp8_adam_step_spec) must store the two-pass step's state bit for bit,
records included, both on steps where a scale changes (its second kernel
recomputes) and on steps where none does, and report which records changed.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import adam as oadam
import tensor_scaled_fp8_amd as tsf
from tests.gpu_util import bf16_bits, f32_bits, to_dev_bf16, u8

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def _ulp_fp16(x):
    a = np.abs(x)
    return np.where(a >= 2.0 ** -14, 2.0 ** (np.floor(np.log2(np.maximum(a, 1e-300))) - 10), 2.0 ** -24)


def _ulp_e4m3(x):
    a = np.abs(x)
    return np.where(a >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(a, 1e-300))) - 3), 2.0 ** -9)


def _near_boundary(amax, fmax):
    if amax == 0 or not math.isfinite(amax):
        return False
    r = math.log2(fmax / amax)
    return abs(r - round(r)) < 1e-5 or abs((r - math.floor(r)) - 1) < 1e-5


def _state_host(st):
    recs = [tsf.read_scale(r) for r in (st.s_m1, st.s_m2, st.s_w)]
    return (u8(st.m1), st.m2.cpu().numpy().view(np.uint16), st.w16.cpu().numpy().view(np.uint16), recs)


def _grad(n, seed, sigma=1e-5):
    g = np.random.Generator(np.random.PCG64(seed))
    gb = oracle.f64_to_bf16_rne(g.standard_normal(n) * sigma)
    s_g = tsf.new_scale(1)[0]
    g8, _ = tsf.fp8_quantize(to_dev_bf16(gb.reshape(16, -1)), "e5m2", s_g, transposed=False)  # n % 256 == 0
    return g8.reshape(-1), s_g


def _check_step(before, after_state, w_bf16, g8, s_g, step):
    m1c, m2b, w16b, (r1, r2, rw) = before
    rg = tsf.read_scale(s_g)
    want = oadam.adam_step(u8(g8), rg["scale_inv"], m1c, r1["scale_inv"], m2b, r2["scale_inv"], w16b, rw["scale_inv"],
                           HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"], step)
    n1, n2, nw = _state_host(after_state)[:3]
    k1, k2, kw = (tsf.read_scale(r) for r in (after_state.s_m1, after_state.s_m2, after_state.s_w))
    for name, kr, wr, fmax in (("m1", k1, want["m1_rec"], 448.0), ("m2", k2, want["m2_rec"], 65504.0),
                               ("w", kw, want["w_rec"], 65504.0)):
        if kr["bias"] != wr["bias"]:
            assert _near_boundary(wr["amax"], fmax), (name, kr["bias"], wr["bias"], wr["amax"])
        assert kr["flags"] == wr["flags"], name
        assert kr["scale_inv"] == 2.0 ** -kr["bias"], name
    g0 = oracle.decode_table(oracle.E5M2)[u8(g8)] * rg["scale_inv"]
    m10 = oracle.decode_table(oracle.E4M3)[m1c] * r1["scale_inv"]
    w0 = oadam.f16_to_f64(w16b) * rw["scale_inv"]
    mag = {"m1": HP["beta1"] * np.abs(m10) + (1 - HP["beta1"]) * np.abs(g0), "m2": want["m2"],
           "w": np.abs(w0) + np.abs(want["w"] - w0)}
    v1 = oracle.decode_table(oracle.E4M3)[n1] * k1["scale_inv"]
    tol1 = _ulp_e4m3(want["m1"] * k1["scale"]) * k1["scale_inv"] + 2e-6 * mag["m1"]
    assert np.all(np.abs(v1 - want["m1"]) <= tol1), ("m1", float(np.max(np.abs(v1 - want["m1"]) / tol1)))
    for name, bits, rec, ref in (("m2", n2, k2, want["m2"]), ("w", nw, kw, want["w"])):
        v = oadam.f16_to_f64(bits) * rec["scale_inv"]
        tol = _ulp_fp16(ref * rec["scale"]) * rec["scale_inv"] + 2e-6 * mag[name]
        assert np.all(np.abs(v - ref) <= tol), (name, float(np.max(np.abs(v - ref) / tol)))
    if w_bf16 is not None:
        wb = oracle.bf16_to_f64(bf16_bits(w_bf16))
        tol = oracle.bf16_ulp(want["w"]) + 2e-6 * mag["w"]
        assert np.all(np.abs(wb - want["w"]) <= tol)


def test_master_init_bit_exact():
    g = np.random.Generator(np.random.PCG64(1))
    wb = oracle.f64_to_bf16_rne(g.standard_normal(272 * 528) * 0.02)
    st = tsf.AdamState(to_dev_bf16(wb))
    want = oadam.master_init(wb)
    assert np.array_equal(st.w16.cpu().numpy().view(np.uint16), want["w16"])
    r = tsf.read_scale(st.s_w)
    assert (r["bias"], r["flags"], f32_bits(r["amax"])) == (want["rec"]["bias"], want["rec"]["flags"],
                                                           f32_bits(want["rec"]["amax"]))
    assert r["reduce_bits"] == 0


@pytest.mark.parametrize("n,sigma_w,sigma_g", [(272 * 528, 0.02, 1e-5), (256, 0.02, 1e-3), (4096 * 16, 0.006, 1e-7),
                                               (784 * 2064, 1.0, 1e-2)])
def test_adam_steps_match_oracle(n, sigma_w, sigma_g):
    g = np.random.Generator(np.random.PCG64(n))
    wb = oracle.f64_to_bf16_rne(g.standard_normal(n) * sigma_w)
    st = tsf.AdamState(to_dev_bf16(wb))
    w_out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    for step in range(1, 4):
        g8, s_g = _grad(n, 100 * step + n, sigma_g)
        before = _state_host(st)
        tsf.fp8_adam_step(st, g8, s_g, w_bf16=w_out, **HP)
        torch.cuda.synchronize()
        _check_step(before, st, w_out, g8, s_g, step)


def test_adam_zero_gradient_and_no_bf16_output():
    n = 4096
    g = np.random.Generator(np.random.PCG64(3))
    wb = oracle.f64_to_bf16_rne(g.standard_normal(n) * 0.05)
    st = tsf.AdamState(to_dev_bf16(wb))
    g8, s_g = _grad(n, 5, 1e-4)
    tsf.fp8_adam_step(st, g8, s_g, **HP)          # moments become non-zero
    zero8 = torch.zeros(n, dtype=torch.uint8, device="cuda")
    s0 = tsf.new_scale(1)[0]
    tsf.fp8_scale_fixed(s0, 0)
    before = _state_host(st)
    tsf.fp8_adam_step(st, zero8, s0, **HP)
    torch.cuda.synchronize()
    _check_step(before, st, None, zero8, s0, 2)


def test_adam_full_size_gpt7b_proj_weight():
    """A full GPT-7B proj weight (4096 x 4096) through one step."""
    n = 4096 * 4096
    g = np.random.Generator(np.random.PCG64(77))
    wb = oracle.f64_to_bf16_rne(g.standard_normal(n) * 0.02)
    st = tsf.AdamState(to_dev_bf16(wb))
    g8, s_g = _grad(n, 78, 1e-5)
    w_out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    before = _state_host(st)
    tsf.fp8_adam_step(st, g8, s_g, w_bf16=w_out, **HP)
    torch.cuda.synchronize()
    _check_step(before, st, w_out, g8, s_g, 1)


def _rec_fields(r):
    d = tsf.read_scale(r)
    return (d["bias"], d["flags"], f32_bits(d["amax"]), d["scale"], d["scale_inv"], d["reduce_bits"])


def _same_state(a, b):
    for x, y in ((a.m1, b.m1), (a.m2, b.m2), (a.w16, b.w16)):
        assert torch.equal(x, y)
    for x, y in ((a.s_m1, b.s_m1), (a.s_m2, b.s_m2), (a.s_w, b.s_w)):
        assert _rec_fields(x) == _rec_fields(y)


@pytest.mark.parametrize("n,sigma_w,sigma_g", [(272 * 528, 0.02, 1e-5), (4096 * 16, 0.5, 1e-3)])
def test_adam_spec_equals_two_pass(n, sigma_w, sigma_g):
    """Ten steps with one fixed gradient: the moments grow geometrically, so
    some steps move a tensor's max across a power of two (the second pass
    runs) and others do not; every step's state, records and bf16 weights
    equal the two-pass step's, and the reported mask equals the records
    whose bias changed."""
    g = np.random.Generator(np.random.PCG64(n + 9))
    wb = to_dev_bf16(oracle.f64_to_bf16_rne(g.standard_normal(n) * sigma_w))
    a, b = tsf.AdamState(wb), tsf.AdamState(wb)
    _same_state(a, b)
    g8, s_g = _grad(n, n + 10, sigma_g)
    wa = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    wbo = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    missed = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    masks = []
    for step in range(1, 11):
        before = [tsf.read_scale(r)["bias"] for r in (b.s_m1, b.s_m2, b.s_w)]
        host_before = _state_host(b)
        tsf.fp8_adam_step(a, g8, s_g, w_bf16=wa, **HP)
        tsf.fp8_adam_step_spec(b, g8, s_g, w_bf16=wbo, missed=missed, **HP)
        torch.cuda.synchronize()
        _same_state(a, b)
        assert torch.equal(wa.view(torch.int16), wbo.view(torch.int16)), step
        after = [tsf.read_scale(r)["bias"] for r in (b.s_m1, b.s_m2, b.s_w)]
        mask = int(missed.item())
        assert mask == sum(1 << i for i in range(3) if before[i] != after[i]), (step, mask, before, after)
        masks.append(mask)
        if step <= 2:
            _check_step(host_before, b, wbo, g8, s_g, step)
    assert masks[0] != 0 and 0 in masks, masks      # both paths taken


def test_adam_spec_full_size_gpt7b_proj_weight():
    """A full GPT-7B proj weight (4096 x 4096): two one-pass steps equal two
    two-pass steps bit for bit."""
    n = 4096 * 4096
    g = np.random.Generator(np.random.PCG64(79))
    wb = to_dev_bf16(oracle.f64_to_bf16_rne(g.standard_normal(n) * 0.02))
    a, b = tsf.AdamState(wb), tsf.AdamState(wb)
    for step in (1, 2):
        g8, s_g = _grad(n, 80 + step, 1e-5)
        tsf.fp8_adam_step(a, g8, s_g, **HP)
        tsf.fp8_adam_step_spec(b, g8, s_g, **HP)
        torch.cuda.synchronize()
        _same_state(a, b)
