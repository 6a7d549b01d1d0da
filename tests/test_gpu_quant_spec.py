"""fp8_quantize_spec: a1 + a2 + a3 in one pass with the bias guessed from the
record's previous call, then a check that recasts when the guess was
wrong, through the C ABI.

[Perez et al. review, "Proposed method", bullets 1-4: the bias comes from
the tensor's own current max |x|.] The guess only decides how much work
is done: after every call the record and every FP8 byte must equal the
oracle's (bit-exact) and what fp8_quantize gives on a separate record.
Sequences mix repeated magnitudes (the guess holds) with changed ones (it
does not), in both formats, with margins and mu; special tensors (NaN,
inf, zeros, empty) and a full-size weight are included."""
import numpy as np
import pytest
import torch

import oracle
from oracle import E4M3, E5M2
import tensor_scaled_fp8_amd as tsf
from tests.gpu_util import to_dev_bf16, u8
from tests.test_gpu_kernels import _check_record
from workloads import draw_normal_bf16

pytestmark = pytest.mark.gpu
FMT = {0: E4M3, 1: E5M2}
NAME = {0: "e4m3", 1: "e5m2"}


def _step(bits, fmt_id, s_spec, s_ref, margin=0, mu=0):
    x = to_dev_bf16(bits)
    q = tsf.fp8_quantize_spec(x, NAME[fmt_id], s_spec, margin, mu)
    q1, _ = tsf.fp8_quantize(x, NAME[fmt_id], s_ref, margin, mu, transposed=False)
    r = tsf.read_scale(s_spec)
    _check_record(r, bits, fmt_id, margin, mu)
    a, b = s_spec.cpu(), s_ref.cpu()
    assert torch.equal(a[:6], b[:6]) and torch.equal(a[7:], b[7:]), (a, b)   # word 6: the guess
    if bits.size:
        rec = oracle.scale_record(bits, FMT[fmt_id], margin, mu)
        assert np.array_equal(u8(q), oracle.cast(bits, FMT[fmt_id], rec["bias"])[0])
        assert torch.equal(q, q1)
    return r["bias"]


@pytest.mark.parametrize("fmt_id,margin,mu", [(0, 0, 0), (1, 0, 2), (0, 1, 0), (1, 1, -1)])
@pytest.mark.parametrize("shape", [(272, 400), (1040, 528), (16, 16)])
def test_spec_sequence_hits_and_misses(fmt_id, margin, mu, shape):
    base = 1.0 if fmt_id == 0 else 1e-5
    # repeated magnitudes keep the bias, x4 / x1e3 / x1e-6 changes it
    factors = [1.0, 1.0, 1.1, 4.0, 4.0, 1e3, 1e-6, 1e-6, 1.0]
    s_spec, s_ref = tsf.new_scale(1)[0], tsf.new_scale(1)[0]
    biases = []
    for k, f in enumerate(factors):
        bits = draw_normal_bf16(700 + 31 * k + shape[0], shape, base * f)
        biases.append(_step(bits, fmt_id, s_spec, s_ref, margin, mu))
    assert len(set(biases)) >= 3          # the sequence did change the bias
    assert any(biases[i] == biases[i + 1] for i in range(len(biases) - 1))   # and kept it


def test_spec_special_tensors():
    n = 256
    base = draw_normal_bf16(21, (n, n), 1.0)
    nan, inf = base.copy(), base.copy()
    nan[3, 5] = 0xFFC1
    inf[200, 7] = 0x7F80
    zeros = np.zeros((n, n), np.uint16)
    for fmt_id in (0, 1):
        s_spec, s_ref = tsf.new_scale(1)[0], tsf.new_scale(1)[0]
        for bits in (base, nan, nan, base, inf, zeros, zeros, base):
            _step(bits, fmt_id, s_spec, s_ref)
    s = tsf.new_scale(1)[0]
    tsf.fp8_quantize_spec(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"), "e4m3", s)
    r = tsf.read_scale(s)
    assert r["amax"] == 0.0 and r["flags"] == tsf.FLAG_ZERO and r["bias"] == 0


def test_spec_interleaved_with_fp8_quantize_on_one_record():
    """The tagged maximum and its epoch stay consistent when the same record
    alternates between the two-pass and the speculative path."""
    s = tsf.new_scale(1)[0]
    for k, sigma in enumerate((1.0, 1.0, 1e-3, 50.0, 50.0, 1e-6)):
        bits = draw_normal_bf16(900 + k, (128, 256), sigma)
        x = to_dev_bf16(bits)
        if k % 2:
            q, _ = tsf.fp8_quantize(x, "e4m3", s, transposed=False)
        else:
            q = tsf.fp8_quantize_spec(x, "e4m3", s)
        _check_record(tsf.read_scale(s), bits, 0, 0, 0)
        rec = oracle.scale_record(bits, E4M3)
        assert np.array_equal(u8(q), oracle.cast(bits, E4M3, rec["bias"])[0]), k


def test_spec_full_size_gpt7b_up_weight():
    """W [4096, 16384] ~ N(0, 0.02), then the same weight scaled by 1.01
    (the bias holds) and by 8 (it changes): each bit-identical to
    fp8_quantize, records bit-exact, first and last 64 rows against the
    oracle's cast."""
    wb = draw_normal_bf16(2_000_000 + 3002, (4096, 16384), 0.02)
    w = to_dev_bf16(wb)
    s_spec, s_ref = tsf.new_scale(1)[0], tsf.new_scale(1)[0]
    for f in (1.0, 1.01, 8.0):
        x = w if f == 1.0 else (w.float() * f).to(torch.bfloat16)
        bits = x.cpu().view(torch.int16).numpy().view(np.uint16)
        q = tsf.fp8_quantize_spec(x, "e4m3", s_spec)
        q1, _ = tsf.fp8_quantize(x, "e4m3", s_ref, transposed=False)
        torch.cuda.synchronize()
        assert torch.equal(q, q1), f
        _check_record(tsf.read_scale(s_spec), bits, 0, 0, 0)
        b = oracle.scale_record(bits, E4M3)["bias"]
        got = u8(q)
        for rows in (slice(0, 64), slice(-64, None)):
            assert np.array_equal(got[rows], oracle.cast(bits[rows], E4M3, b)[0]), (f, rows)
