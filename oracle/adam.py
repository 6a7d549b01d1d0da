"""O2 precision-decoupled Adam step, plain float64 (test infrastructure only).

[FP8-LM reading note, "Proposed method", O2] the optimizer keeps its first
moment in FP8, its second moment in FP16 and the master weights in FP16 with
tensor scaling. Readings where the page is silent (the same ones the HIP
path takes): the first moment is E4M3 with a per-tensor power-of-two scale;
the FP16 tensors each carry a per-tensor power-of-two scale chosen like the
FP8 ones with the FP16 maximum 65504; the update is AdamW with bias
correction; every new scale comes from the new tensor's max |value|.

A stored tensor's value is dec(code) * scale_inv of its record. numpy's
float64 -> float16 conversion (round to nearest even) serves as the FP16
encoder; the FP8 encoder and the bias rule are the oracle's own."""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np

from .bf16 import bf16_to_f64, f64_to_bf16_rne
from .formats import E4M3, E5M2, decode_table, encode
from .scaling import compute_bias

FP16_MAX = 65504.0
FP16_STORE = SimpleNamespace(name="fp16", max_finite=FP16_MAX)   # range for the bias rule


def f16_to_f64(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f64_to_f16_rne(x) -> np.ndarray:
    """IEEE binary16 bit patterns, round to nearest even (numpy's conversion)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def _record(amax_value: float, fmt) -> dict:
    b, flags = compute_bias(amax_value, fmt)
    return {"amax": amax_value, "bias": b, "scale": 2.0 ** b, "scale_inv": 2.0 ** -b, "flags": flags}


def _amax(x: np.ndarray) -> float:
    if x.size == 0:
        return 0.0
    if np.isnan(x).any():
        return float("nan")
    return float(np.abs(x).max())


def master_init(w_bf16_bits) -> dict:
    """FP16 master weights from bf16 weights: bits and record."""
    w = bf16_to_f64(w_bf16_bits)
    rec = _record(_amax(w), FP16_STORE)
    return {"w16": f64_to_f16_rne(np.ldexp(w, rec["bias"])), "rec": rec}


def adam_update(g, m1, m2, w, lr, beta1, beta2, eps, weight_decay, step):
    """AdamW with bias correction on float64 arrays: (m1', m2', w')."""
    m1n = beta1 * m1 + (1.0 - beta1) * g
    m2n = beta2 * m2 + (1.0 - beta2) * g * g
    mh = m1n / (1.0 - beta1 ** step)
    vh = m2n / (1.0 - beta2 ** step)
    wn = w - lr * (mh / (np.sqrt(vh) + eps) + weight_decay * w)
    return m1n, m2n, wn


def adam_step(g_codes, g_scale_inv, m1_codes, m1_scale_inv, m2_bits, m2_scale_inv, w16_bits, w_scale_inv,
              lr, beta1, beta2, eps, weight_decay, step) -> dict:
    """One O2 step from stored tensors (codes / FP16 bits and their records'
    scale_inv); returns the new float64 values, the new stored tensors and
    their records, and the new weights rounded to bf16."""
    g = decode_table(E5M2)[np.asarray(g_codes)] * g_scale_inv
    m1 = decode_table(E4M3)[np.asarray(m1_codes)] * m1_scale_inv
    m2 = f16_to_f64(m2_bits) * m2_scale_inv
    w = f16_to_f64(w16_bits) * w_scale_inv
    m1n, m2n, wn = adam_update(g, m1, m2, w, lr, beta1, beta2, eps, weight_decay, step)
    r1, r2, rw = _record(_amax(m1n), E4M3), _record(_amax(m2n), FP16_STORE), _record(_amax(wn), FP16_STORE)
    return {
        "m1": m1n, "m2": m2n, "w": wn,
        "m1_codes": encode(np.ldexp(m1n, r1["bias"]), E4M3), "m1_rec": r1,
        "m2_bits": f64_to_f16_rne(np.ldexp(m2n, r2["bias"])), "m2_rec": r2,
        "w16": f64_to_f16_rne(np.ldexp(wn, rw["bias"])), "w_rec": rw,
        "w_bf16": f64_to_bf16_rne(wn),
    }
