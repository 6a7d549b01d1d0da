"""Host-side checks of the C ABI (no GPU needed, no kernel launched):
the library loads, exports every function include/fp8lin.h declares, the
host copy of the scale rule equals the oracle's bias for every bf16 amax,
and argument validation returns the documented status before any launch."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import tensor_scaled_fp8_amd as tsf
from tensor_scaled_fp8_amd import _lib
from oracle import E4M3, E5M2, FLAG_CLAMPED, bf16_to_f64, compute_bias

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8lin.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(fp8_\w+)\s*\(", src, flags=re.M)))


def test_header_functions_all_exported():
    lib = tsf.load()
    names = _declared_functions()
    assert len(names) >= 11, names
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, f"binding lacks {n}"
    assert lib.fp8_abi_version() == 13


def test_status_strings():
    lib = tsf.load()
    for s in range(4):
        assert lib.fp8_status_str(s)
    assert lib.fp8_status_str(99) == b"unknown status"


@pytest.mark.parametrize("fmt,name", [(E4M3, "e4m3"), (E5M2, "e5m2")])
def test_host_bias_rule_matches_oracle_all_bf16(fmt, name):
    vals = bf16_to_f64(np.arange(0, 0x7F81, dtype=np.uint16))
    for margin, mu in ((0, 0), (1, 0), (0, 3), (-2, -1)):
        for a in vals:
            b, f = tsf.fp8_bias_host(float(a), name, margin, mu)
            rb, rf = compute_bias(float(a), fmt, margin, mu)
            assert (b, f) == (rb, rf), (name, a, margin, mu, b, f, rb, rf)


def test_host_bias_rule_fp32_amax_and_nan():
    g = np.random.Generator(np.random.PCG64(1))
    bits = g.integers(1, 0x7F800000, size=20000, dtype=np.uint32)
    for a in bits.view(np.float32):
        for fmt, name in ((E4M3, "e4m3"), (E5M2, "e5m2")):
            assert tsf.fp8_bias_host(float(a), name) == compute_bias(float(a), fmt)
    assert tsf.fp8_bias_host(math.nan, "e4m3") == (0, 1)
    assert tsf.fp8_bias_host(math.inf, "e5m2") == (0, 1)
    assert tsf.fp8_bias_host(-3.0, "e4m3") == compute_bias(3.0, E4M3)


def _vp(x):
    return ctypes.c_void_p(x)


def test_argument_validation_without_launch():
    lib = tsf.load()
    ok = 4096                          # a 16-byte aligned non-null fake address (never dereferenced)
    INV, UNS = _lib.FP8_ERR_INVALID, _lib.FP8_ERR_UNSUPPORTED
    # null / misaligned / negative / bad enum -> INVALID
    assert lib.fp8_amax(_vp(ok), -1, _vp(ok), None) == INV
    assert lib.fp8_amax(_vp(ok), 10, None, None) == INV
    assert lib.fp8_amax(_vp(ok + 2), 10, _vp(ok), None) == INV
    assert lib.fp8_scale(7, 0, 0, _vp(ok), None) == INV
    assert lib.fp8_scale(0, 5000, 0, _vp(ok), None) == INV
    assert lib.fp8_amax_scale(_vp(ok), 8, 0, 0, -2000, _vp(ok), None) == INV
    assert lib.fp8_scale_reset(_vp(ok + 8), 1, None) == INV
    q = lib.fp8_quantize
    assert q(_vp(ok), 32, 40, 0, 0, 0, _vp(ok), _vp(ok), None, None) == UNS
    assert q(_vp(ok), 32, 32, 2, 0, 0, _vp(ok), _vp(ok), None, None) == INV
    assert q(_vp(ok), 32, 32, 0, 0, 9999, _vp(ok), _vp(ok), None, None) == INV
    assert q(None, 32, 32, 0, 0, 0, _vp(ok), _vp(ok), None, None) == INV
    assert q(_vp(ok), 32, 32, 1, 0, 0, None, _vp(ok), None, None) == INV
    # cast: dims must be multiples of 16
    assert lib.fp8_cast(_vp(ok), 17, 32, 0, _vp(ok), _vp(ok), None, None) == UNS
    assert lib.fp8_cast(_vp(ok), 32, 40, 1, _vp(ok), _vp(ok), None, None) == UNS
    assert lib.fp8_cast(None, 32, 32, 0, _vp(ok), _vp(ok), None, None) == INV
    assert lib.fp8_cast(_vp(ok), 32, 32, 0, _vp(ok), _vp(ok + 4), None, None) == INV
    # gemm
    g = lib.fp8_gemm_nt
    assert g(_vp(ok), 0, _vp(ok), _vp(ok), 0, _vp(ok), 16, 16, 24, _vp(ok), None) == UNS
    assert g(_vp(ok), 0, _vp(ok), _vp(ok), 3, _vp(ok), 16, 16, 16, _vp(ok), None) == INV
    assert g(_vp(ok), 0, None, _vp(ok), 0, _vp(ok), 16, 16, 16, _vp(ok), None) == INV
    assert g(_vp(ok), 0, _vp(ok), _vp(ok), 0, _vp(ok), -16, 16, 16, _vp(ok), None) == INV
    assert g(_vp(ok), 0, _vp(ok), None, 0, _vp(ok), 16, 16, 16, _vp(ok), None) == INV
    gl = lib.fp8_gemm
    assert gl(_vp(ok), 0, 2, _vp(ok), _vp(ok), 0, 0, _vp(ok), 16, 16, 16, _vp(ok), None) == INV
    assert gl(_vp(ok), 0, 0, _vp(ok), _vp(ok), 0, -1, _vp(ok), 16, 16, 16, _vp(ok), None) == INV
    assert gl(_vp(ok), 0, 1, _vp(ok), _vp(ok), 0, 1, _vp(ok), 16, 16, 40, _vp(ok), None) == UNS
    assert gl(_vp(ok), 0, 1, _vp(ok), None, 0, 1, _vp(ok), 16, 16, 16, _vp(ok), None) == INV
    # gemm pair: each argument set checked as fp8_gemm checks it, nothing enqueued on failure
    gp = lib.fp8_gemm_pair
    good = _lib.GemmArgs(ok, 1, 0, ok, ok, 0, 0, ok, 16, 16, 16, ok)
    assert gp(None, ctypes.byref(good), None) == INV
    assert gp(ctypes.byref(good), None, None) == INV
    bad_fmt = _lib.GemmArgs(ok, 2, 0, ok, ok, 0, 0, ok, 16, 16, 16, ok)
    assert gp(ctypes.byref(good), ctypes.byref(bad_fmt), None) == INV
    bad_layout = _lib.GemmArgs(ok, 0, 3, ok, ok, 1, 1, ok, 16, 16, 16, ok)
    assert gp(ctypes.byref(bad_layout), ctypes.byref(good), None) == INV
    ragged = _lib.GemmArgs(ok, 0, 1, ok, ok, 1, 1, ok, 16, 16, 40, ok)
    assert gp(ctypes.byref(good), ctypes.byref(ragged), None) == UNS
    misaligned = _lib.GemmArgs(ok, 0, 1, ok, ok, 1, 1, ok, 16, 16, 16, ok + 2)
    assert gp(ctypes.byref(good), ctypes.byref(misaligned), None) == INV
    no_rec = _lib.GemmArgs(ok, 0, 1, None, ok, 1, 1, ok, 16, 16, 16, ok)
    assert gp(ctypes.byref(no_rec), ctypes.byref(good), None) == INV
    # workspace GEMM: fp8_gemm's checks plus an aligned workspace; workspace size rule
    gw = lib.fp8_gemm_ws
    assert gw(_vp(ok), 0, 0, _vp(ok), _vp(ok), 0, 1, _vp(ok), 16, 16, 24, _vp(ok), 0, _vp(ok), 1 << 20, None) == UNS
    assert gw(_vp(ok), 0, 0, _vp(ok), _vp(ok), 0, 1, _vp(ok), 16, 16, 16, _vp(ok), 0, _vp(ok + 8), 1 << 20,
              None) == INV
    assert gw(_vp(ok), 0, 0, None, _vp(ok), 0, 1, _vp(ok), 16, 16, 16, _vp(ok), 0, None, 0, None) == INV
    assert gw(_vp(ok), 0, 0, _vp(ok), _vp(ok), 0, 1, _vp(ok), 16, 16, 16, _vp(ok), 3, None, 0, None) == INV
    # no-allocation GEMM: fp8_gemm's checks and the split enum, before any device access
    gn = lib.fp8_gemm_noalloc
    assert gn(_vp(ok), 0, 0, _vp(ok), _vp(ok), 0, 1, _vp(ok), 16, 16, 24, _vp(ok), 0, None) == UNS
    assert gn(_vp(ok), 0, 0, None, _vp(ok), 0, 1, _vp(ok), 16, 16, 16, _vp(ok), 0, None) == INV
    assert gn(_vp(ok), 0, 0, _vp(ok), _vp(ok), 0, 1, _vp(ok), 16, 16, 16, _vp(ok), 3, None) == INV
    assert gn(_vp(ok), 0, 2, _vp(ok), _vp(ok), 0, 1, _vp(ok), 16, 16, 16, _vp(ok), 0, None) == INV
    assert gn(_vp(ok), 0, 0, _vp(ok), _vp(ok), 0, 1, _vp(ok), 16, 16, 16, _vp(ok + 2), 0, None) == INV
    assert _lib.FP8_NOALLOC_SCRATCH_BYTES == 128 * 2 * 65536 * 4
    wb = lib.fp8_gemm_workspace_bytes
    TAIL, AUTO, NEVER = _lib.FP8_SPLIT_TAIL, _lib.FP8_SPLIT_AUTO, _lib.FP8_SPLIT_NEVER
    assert wb(0, 0, 256, 256, 1024, TAIL) == 2 * 65536 * 4      # one tile: its two halves' FP32 partials
    assert wb(0, 0, 784, 272, 2048, TAIL) == 8 * 2 * 65536 * 4  # 4 x 2 tiles
    assert wb(0, 0, 256, 256, 1024, AUTO) == 0                  # too short a reduction to pay
    assert wb(0, 0, 256, 256, 16384, AUTO) == 2 * 65536 * 4
    assert wb(0, 0, 256, 256, 16384, NEVER) == 0
    assert wb(1, 0, 256, 256, 1024, TAIL) == 0                  # backward formats never split
    assert wb(0, 1, 256, 256, 1024, TAIL) == 0
    assert wb(0, 0, 256, 256, 256, TAIL) == 0                   # R below 512
    assert wb(0, 0, 256, 256, 1040, TAIL) == 0                  # R not a multiple of 256
    assert wb(0, 0, -16, 256, 1024, TAIL) == 0
    assert lib.fp8_linear_scratch_bytes(256, 16384, 256) == 2 * 65536 * 4
    assert lib.fp8_linear_scratch_bytes(256, 1024, 256) == 0
    # speculative quantise: fp8_quantize's checks, row-major output required
    qs = lib.fp8_quantize_spec
    assert qs(_vp(ok), 16, 16, 0, 0, 0, _vp(ok), None, None) == INV
    assert qs(_vp(ok), 16, 24, 0, 0, 0, _vp(ok), _vp(ok), None) == UNS
    assert qs(_vp(ok), 16, 16, 2, 0, 0, _vp(ok), _vp(ok), None) == INV
    assert qs(_vp(ok), 16, 16, 0, 0, 0, None, _vp(ok), None) == INV
    assert qs(_vp(ok), 16, 16, 0, 0, 0, _vp(ok), _vp(ok + 4), None) == INV
    # quantize batch: 1..4 argument sets, each checked as fp8_quantize's, distinct records
    qb = lib.fp8_quantize_batch
    QA = _lib.QuantizeArgs
    one = (QA * 1)(QA(ok, 16, 16, 0, 0, 0, ok, ok, None))
    assert qb(None, 1, None) == INV
    assert qb(one, 0, None) == INV
    five = (QA * 5)(*[QA(ok, 16, 16, 0, 0, 0, ok + 64 * i, ok, None) for i in range(5)])
    assert qb(five, 5, None) == INV
    dup = (QA * 2)(QA(ok, 16, 16, 0, 0, 0, ok, ok, None), QA(ok, 16, 16, 1, 0, 0, ok, ok, None))
    assert qb(dup, 2, None) == INV
    bad = (QA * 2)(QA(ok, 16, 16, 0, 0, 0, ok, ok, None), QA(ok, 16, 24, 1, 0, 0, ok + 64, ok, None))
    assert qb(bad, 2, None) == UNS
    bad = (QA * 2)(QA(ok, 16, 16, 0, 0, 0, ok, ok, None), QA(ok, 16, 16, 2, 0, 0, ok + 64, ok, None))
    assert qb(bad, 2, None) == INV
    bad = (QA * 2)(QA(ok, 16, 16, 0, 0, 0, ok, ok, None), QA(ok, 16, 16, 1, 0, 0, ok + 64, ok + 3, None))
    assert qb(bad, 2, None) == INV
    bad = (QA * 1)(QA(ok, 16, 16, 0, 5000, 0, ok, ok, None))
    assert qb(bad, 1, None) == INV
    # linear: workspace checks
    ws = _lib.LinearWs(ok, ok, ok, ok, ok, ok, ok, ok, ok)
    assert lib.fp8_linear_fwd(_vp(ok), _vp(ok), 16, 16, 16, 0, None, _vp(ok), None) == INV
    assert lib.fp8_linear_fwd(_vp(ok), _vp(ok), 16, 24, 16, 0, ctypes.byref(ws), _vp(ok), None) == UNS
    ws_bad = _lib.LinearWs(ok, ok, ok, ok, None, ok, ok, ok, ok)
    assert lib.fp8_linear_bwd(_vp(ok), 16, 16, 16, 0, 0, ctypes.byref(ws_bad), None, None, None) == INV
    # the transposed copies are optional, but aligned when given
    ws_mis = _lib.LinearWs(ok, ok + 4, ok, None, ok, None, ok, ok, ok)
    assert lib.fp8_linear_fwd(_vp(ok), _vp(ok), 16, 16, 16, 0, ctypes.byref(ws_mis), _vp(ok), None) == INV
    # X and W quantised in one batch: their records must differ
    ws_same = _lib.LinearWs(ok, None, ok, None, ok, None, ok, ok, ok + 64)
    assert lib.fp8_linear_fwd(_vp(ok), _vp(ok), 16, 16, 16, 0, ctypes.byref(ws_same), _vp(ok), None) == INV
    # the forward's scratch is optional, but aligned when given
    ws_scr = _lib.LinearWs(ok, None, ok, None, ok, None, ok, ok + 64, ok + 128, ok + 8, 1 << 20)
    assert lib.fp8_linear_fwd(_vp(ok), _vp(ok), 16, 16, 16, 0, ctypes.byref(ws_scr), _vp(ok), None) == INV
    # the backward's dY record must differ from X's and W's (its quantise rewrites it)
    for sdy in (ok, ok + 64):
        ws_dy = _lib.LinearWs(ok, None, ok, None, ok, None, ok, ok + 64, sdy)
        assert lib.fp8_linear_bwd(_vp(ok), 16, 16, 16, 0, 0, ctypes.byref(ws_dy), _vp(ok), _vp(ok), None) == INV
    ws_nox = _lib.LinearWs(None, None, ok, None, ok, None, ok, ok, ok)
    assert lib.fp8_linear_fwd(_vp(ok), _vp(ok), 16, 16, 16, 0, ctypes.byref(ws_nox), _vp(ok), None) == INV
    # fixed bias: only [-126, 126]
    assert lib.fp8_scale_fixed(_vp(ok), 127, None) == INV
    assert lib.fp8_scale_fixed(_vp(ok), -127, None) == INV
    assert lib.fp8_scale_fixed(None, 0, None) == INV
    assert lib.fp8_scale_fixed(_vp(ok + 4), 0, None) == INV
    # cached-weight forward
    c = lib.fp8_linear_fwd_cached
    args = lambda **kw: [kw.get(k, d) for k, d in (
        ("X", _vp(ok)), ("M", 16), ("K", 16), ("N", 16), ("margin", 0), ("mode", 0), ("w8t", _vp(ok)),
        ("lw", 1), ("sw", _vp(ok)), ("x8", _vp(ok)), ("sx", _vp(ok + 64)), ("Y", _vp(ok)), ("st", None))]
    assert c(*args(mode=2)) == INV
    assert c(*args(lw=2)) == INV
    assert c(*args(lw=-1)) == INV
    assert c(*args(K=24)) == UNS
    assert c(*args(sw=None)) == INV
    assert c(*args(sx=_vp(ok + 8))) == INV
    assert c(*args(x8=None)) == INV
    assert c(*args(w8t=None)) == INV
    assert c(*args(Y=_vp(ok + 2))) == INV
    assert c(*args(margin=-5000)) == INV
    assert c(*args(sx=_vp(ok))) == INV                  # X's record shared with W's
    assert c(*args(sx=_vp(ok), mode=1)) == INV
    # FP8 weight gradient
    wg = lib.fp8_wgrad_fp8
    wargs = lambda **kw: [kw.get(k, d) for k, d in (
        ("x8", _vp(ok)), ("lx", 0), ("sx", _vp(ok)), ("dy8", _vp(ok)), ("ldy", 1), ("sdy", _vp(ok)), ("K", 16),
        ("N", 16),
        ("M", 16), ("margin", 0), ("mu", 0), ("dW", _vp(ok)), ("s_dw", _vp(ok)), ("dw8", _vp(ok)),
        ("dw8t", None), ("st", None))]
    assert wg(*wargs(M=24)) == UNS
    assert wg(*wargs(K=-16)) == INV
    assert wg(*wargs(s_dw=None)) == INV
    assert wg(*wargs(dw8=None)) == INV
    assert wg(*wargs(dW=_vp(ok + 2))) == INV
    assert wg(*wargs(dw8t=_vp(ok + 1))) == INV
    assert wg(*wargs(mu=3000)) == INV
    assert wg(*wargs(x8=None)) == INV
    assert wg(*wargs(lx=2)) == INV
    assert wg(*wargs(ldy=-1)) == INV
    # O2 Adam
    ad = lib.fp8_adam_step
    aargs = lambda **kw: [kw.get(k, d) for k, d in (
        ("n", 64), ("g8", _vp(ok)), ("s_g", _vp(ok)), ("m1", _vp(ok)), ("s_m1", _vp(ok)), ("m2", _vp(ok)),
        ("s_m2", _vp(ok)), ("w", _vp(ok)), ("s_w", _vp(ok)), ("wb", None), ("lr", 1e-3), ("b1", 0.9),
        ("b2", 0.95), ("eps", 1e-8), ("wd", 0.1), ("step", 1), ("st", None))]
    assert ad(*aargs(n=40)) == UNS
    assert ad(*aargs(step=0)) == INV
    assert ad(*aargs(b1=1.0)) == INV
    assert ad(*aargs(b2=-0.1)) == INV
    assert ad(*aargs(eps=0.0)) == INV
    assert ad(*aargs(wd=-1.0)) == INV
    assert ad(*aargs(lr=math.inf)) == INV
    assert ad(*aargs(lr=math.nan)) == INV
    assert ad(*aargs(s_m2=None)) == INV
    assert ad(*aargs(m1=_vp(ok + 8))) == INV
    assert ad(*aargs(wb=_vp(ok + 2))) == INV
    # one-pass Adam (out of place): the same checks, plus the outputs
    # present, aligned and disjoint from the inputs and from each other
    sp = lib.fp8_adam_step_spec
    base = {"g8": 0, "m1": 0x1000, "m2": 0x2000, "w": 0x3000, "m1o": 0x4000, "m2o": 0x5000, "wo": 0x6000,
            "wb": 0x7000}
    sargs = lambda **kw: [kw.get(k, d) for k, d in (
        ("n", 64), ("g8", _vp(ok + base["g8"])), ("s_g", _vp(ok)), ("m1", _vp(ok + base["m1"])),
        ("m2", _vp(ok + base["m2"])), ("w", _vp(ok + base["w"])), ("m1o", _vp(ok + base["m1o"])),
        ("m2o", _vp(ok + base["m2o"])), ("wo", _vp(ok + base["wo"])), ("s_m1", _vp(ok)), ("s_m2", _vp(ok)),
        ("s_w", _vp(ok)), ("wb", None), ("missed", None), ("lr", 1e-3), ("b1", 0.9), ("b2", 0.95),
        ("eps", 1e-8), ("wd", 0.1), ("step", 1), ("st", None))]
    assert sp(*sargs(n=40)) == UNS
    assert sp(*sargs(step=0)) == INV
    assert sp(*sargs(eps=0.0)) == INV
    assert sp(*sargs(s_w=None)) == INV
    assert sp(*sargs(m2o=None)) == INV
    assert sp(*sargs(wo=_vp(ok + base["wo"] + 8))) == INV
    assert sp(*sargs(missed=_vp(ok + 2))) == INV
    assert sp(*sargs(m1o=_vp(ok + base["m1"]))) == INV                 # in place
    assert sp(*sargs(m2o=_vp(ok + base["w"] + 64))) == INV             # overlaps the weights read
    assert sp(*sargs(wo=_vp(ok + base["m2o"] + 64))) == INV            # overlaps another output
    assert sp(*sargs(wb=_vp(ok + base["m1o"]))) == INV                 # bf16 weights over m1_out
    assert sp(*sargs(g8=_vp(ok + base["wo"] + 112))) == INV            # gradient read inside w16_out
    im = lib.fp8_adam_init_master
    assert im(40, _vp(ok), _vp(ok), _vp(ok), None) == UNS
    assert im(64, None, _vp(ok), _vp(ok), None) == INV
    assert im(64, _vp(ok), _vp(ok), None, None) == INV


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(16, 16, dtype=torch.bfloat16)
    s = torch.zeros(8, dtype=torch.int32)
    with pytest.raises(ValueError, match="device tensor"):
        tsf.fp8_amax(x, s)
