"""Seeded synthetic inputs for the per-tensor scaled FP8 linear.

This module is shared by the oracle side and the HIP side. It holds the
layer shapes and draws random bf16 bit patterns; it contains none of the
method's arithmetic (no amax, no scale rule, no FP8 encoding, no GEMM).

Shapes and distributions: one transformer layer's linears per workload,
tokens x in -> out, with X ~ N(0, 1), W ~ N(0, sigma_w), dY ~ N(0, sigma_dy)
(sigma is the standard deviation). The Llama-2-70B-style workload adds
outlier input channels (x100) and log-uniform gradient magnitudes.

Every tensor is drawn from numpy's PCG64 generator in float32 and rounded to
bf16 with round-to-nearest-even; the seed of a tensor is
1_000_000 * workload + 1000 * linear_index + {X: 1, W: 2, dY: 3}.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "Linear", "Workload", "WORKLOADS", "workload", "f32_to_bf16_bits",
    "draw_normal_bf16", "linear_inputs", "random_bf16_bits",
]


@dataclass(frozen=True)
class Linear:
    name: str
    M: int            # tokens
    K: int            # in features
    N: int            # out features
    x_seed_linear: Optional[int] = None   # reuse another linear's X (shared input)


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    linears: List[Linear]
    sigma_w: float
    sigma_dy: float
    margin: int = 0
    mu_log2: int = 0
    x_outliers: bool = False       # 0.1% of input channels scaled by 100
    dy_log_uniform: bool = False   # |dY| = 2^U, U ~ Uniform[-30, -8), random sign
    notes: str = ""

    def flops_fwd_bwd(self) -> int:
        return sum(6 * l.M * l.K * l.N for l in self.linears)

    def quant_bytes(self, transposed: bool = False) -> int:
        """HBM bytes of amax (2 B/elem read) + cast (2 B read, 1 B written per
        FP8 copy) over X, W and dY of every linear: 5 B per element for the
        row-major copy alone, 6 B with the transposed copy as well."""
        per = 6 if transposed else 5
        return sum(per * (l.M * l.K + l.K * l.N + l.M * l.N) for l in self.linears)


def _layer(index, name, M, d, qkv_out, mlp, sigma_w, sigma_dy, margin=0):
    return Workload(
        index=index, name=name,
        linears=[Linear("qkv", M, d, qkv_out), Linear("proj", M, d, d),
                 Linear("up", M, d, mlp), Linear("down", M, mlp, d)],
        sigma_w=sigma_w, sigma_dy=sigma_dy, margin=margin)


WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "gpt125m-mlp-up", [Linear("up", 512, 768, 3072)],
                sigma_w=0.02, sigma_dy=1e-4),
    2: _layer(2, "gpt7b-layer", 4096, 4096, 12288, 16384, 0.02, 1e-5),
    3: _layer(3, "gpt13b-layer", 8192, 5120, 15360, 20480, 0.02, 1e-5, margin=1),
    4: _layer(4, "gpt175b-layer", 2048, 12288, 36864, 49152, 0.006, 1e-5),
    5: Workload(
        5, "llama2-70b-swiglu-layer",
        [Linear("qkv", 4096, 8192, 10240), Linear("gate", 4096, 8192, 28672),
         Linear("up", 4096, 8192, 28672, x_seed_linear=1),
         Linear("down", 4096, 28672, 8192)],
        sigma_w=0.02, sigma_dy=0.0, x_outliers=True, dy_log_uniform=True,
        notes="gate and up read the same X (the up linear reuses the gate's X seed)"),
}


def workload(index: int) -> Workload:
    return WORKLOADS[index]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (NaN kept quiet)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def draw_normal_bf16(seed: int, shape, sigma: float) -> np.ndarray:
    g = _rng(seed)
    a = g.standard_normal(int(np.prod(shape)), dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return f32_to_bf16_bits(a).reshape(shape)


def random_bf16_bits(seed: int, shape, finite_only: bool = True) -> np.ndarray:
    """Uniformly random bf16 bit patterns (every exponent, both signs)."""
    g = _rng(seed)
    bits = g.integers(0, 1 << 16, size=int(np.prod(shape)), dtype=np.uint32).astype(np.uint16)
    if finite_only:
        bad = (bits & 0x7F80) == 0x7F80
        bits[bad] &= 0xBFFF  # clear the top exponent bit: finite again
    return bits.reshape(shape)


def _seed(wl: Workload, li: int, which: int) -> int:
    return 1_000_000 * wl.index + 1000 * li + which


def linear_inputs(wl: Workload, li: int, rows_x: Optional[int] = None):
    """(X bits [M,K], W bits [K,N], dY bits [M,N]) as uint16 arrays.

    rows_x limits the number of token rows (a leading slice of the full
    tensors, drawn from the same stream), for bounded CPU samples."""
    lin = wl.linears[li]
    M = lin.M if rows_x is None else min(rows_x, lin.M)
    xl = li if lin.x_seed_linear is None else lin.x_seed_linear
    # X: N(0, 1), drawn row-major; a leading row slice reads a stream prefix.
    g = _rng(_seed(wl, xl, 1))
    x = g.standard_normal(M * lin.K, dtype=np.float32).reshape(M, lin.K)
    if wl.x_outliers:
        go = _rng(_seed(wl, xl, 1) + 500)
        n_out = int(round(0.001 * lin.K))
        ch = go.choice(lin.K, size=n_out, replace=False)
        x[:, ch] *= np.float32(100.0)
    X = f32_to_bf16_bits(x)
    del x
    W = draw_normal_bf16(_seed(wl, li, 2), (lin.K, lin.N), wl.sigma_w)
    if wl.dy_log_uniform:
        g = _rng(_seed(wl, li, 3))
        u = g.uniform(-30.0, -8.0, size=M * lin.N).astype(np.float32)
        s = np.where(g.integers(0, 2, size=M * lin.N) == 0, np.float32(1), np.float32(-1))
        dy = (s * np.exp2(u)).astype(np.float32).reshape(M, lin.N)
        dY = f32_to_bf16_bits(dy)
    else:
        g = _rng(_seed(wl, li, 3))
        dy = g.standard_normal(M * lin.N, dtype=np.float32)
        dy *= np.float32(wl.sigma_dy)
        dY = f32_to_bf16_bits(dy).reshape(M, lin.N)
    return X, W, dY
