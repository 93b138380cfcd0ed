"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

A package of its own, outside the library and the oracle, so that both sides
take the same arrays without either importing the other.  It only *draws*
inputs: Gaussian weights with a few scaled-up input
channels (outliers) and Gaussian activations, rounded to bf16.  It holds none
of the quantization or matmul arithmetic; both the CPU oracle and the GPU path
receive the same arrays from here.

Shapes follow the Llama-3-8B projection matrices the quantization pages use as
their running 8B example (qkv, o, gate_up, down), stored as ``[N, K]`` = out x
in so that ``Y = X W^T`` (vLLM quantization page, section 2, linear layer).

All randomness is numpy's PCG64 ``default_rng(seed)``; bf16 values are kept as
``uint16`` bit patterns (round-to-nearest-even from float32).
"""
from __future__ import annotations

import numpy as np

# [N, K] of the four projections of one Llama-3-8B layer.
LLAMA3_8B_SHAPES = {
    "qkv": (6144, 4096),
    "o": (4096, 4096),
    "gate_up": (28672, 4096),
    "down": (4096, 14336),
}
SHAPE_ORDER = ("qkv", "o", "gate_up", "down")


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def weights(n: int, k: int, seed: int, std: float = 0.02,
            outlier_frac: float = 0.001, outlier_gain: float = 20.0,
            outlier_cols=None):
    """Weight matrix ``[n, k]`` ~ N(0, std) with some input channels scaled.

    ``outlier_cols`` fixes the scaled channels; otherwise ``round(outlier_frac*k)``
    distinct channels are drawn with the same generator after the Gaussian draw.
    Returns ``(w_bf16_bits, outlier_cols)``.
    """
    rng = np.random.default_rng(seed)
    w = rng.normal(0.0, std, size=(n, k)).astype(np.float32)
    if outlier_cols is None:
        n_out = int(round(outlier_frac * k))
        outlier_cols = np.sort(rng.choice(k, n_out, replace=False)) if n_out else np.zeros(0, np.int64)
    outlier_cols = np.asarray(outlier_cols, dtype=np.int64)
    if outlier_cols.size:
        w[:, outlier_cols] *= np.float32(outlier_gain)
    return f32_to_bf16_bits(w), outlier_cols


def activations(m: int, k: int, seed: int, n_outlier_channels: int = 0,
                outlier_gain: float = 50.0):
    """Activations ``[m, k]`` ~ N(0, 1), optionally with channels scaled up.

    Returns ``(x_bf16_bits, outlier_cols)``.
    """
    rng = np.random.default_rng(seed)
    x = rng.normal(0.0, 1.0, size=(m, k)).astype(np.float32)
    cols = np.zeros(0, np.int64)
    if n_outlier_channels:
        cols = np.sort(rng.choice(k, n_outlier_channels, replace=False))
        x[:, cols] *= np.float32(outlier_gain)
    return f32_to_bf16_bits(x), cols


def activations_f16(m: int, k: int, seed: int, n_outlier_channels: int = 0,
                    outlier_gain: float = 50.0):
    """As ``activations`` but rounded to fp16 (nearest even); returns
    ``(x_fp16_bits, outlier_cols)``."""
    rng = np.random.default_rng(seed)
    x = rng.normal(0.0, 1.0, size=(m, k)).astype(np.float32)
    cols = np.zeros(0, np.int64)
    if n_outlier_channels:
        cols = np.sort(rng.choice(k, n_outlier_channels, replace=False))
        x[:, cols] *= np.float32(outlier_gain)
    return x.astype(np.float16).view(np.uint16), cols


def tiny_reference():
    """Tiny case: W [256, 512] ~ N(0, 0.02), input channels 7 and 300 scaled x50,
    X [1, 512] ~ N(0, 1); one generator (seed 0), W drawn first, then X."""
    rng = np.random.default_rng(0)
    w = rng.normal(0.0, 0.02, size=(256, 512)).astype(np.float32)
    w[:, [7, 300]] *= np.float32(50.0)
    x = rng.normal(0.0, 1.0, size=(1, 512)).astype(np.float32)
    return f32_to_bf16_bits(w), f32_to_bf16_bits(x)


def decode_case(name: str, m: int = 1):
    """Decode-GEMV inputs for one projection: weight seed 1000+i, activation seed 2000+i."""
    i = SHAPE_ORDER.index(name)
    n, k = LLAMA3_8B_SHAPES[name]
    w, _ = weights(n, k, seed=1000 + i)
    x, _ = activations(m, k, seed=2000 + i)
    return w, x


def prefill_case(name: str, m: int = 2048):
    """Prefill-GEMM inputs: weights as the decode case, X [m, K] ~ N(0,1) with
    4 channels scaled x50 (seed 3000+i)."""
    i = SHAPE_ORDER.index(name)
    n, k = LLAMA3_8B_SHAPES[name]
    w, _ = weights(n, k, seed=1000 + i)
    x, _ = activations(m, k, seed=3000 + i, n_outlier_channels=4)
    return w, x


def q4k_case(name: str, m: int = 1):
    """Super-block format inputs: weights seed 4000+i (recipe as decode), X seed 2000+i."""
    i = SHAPE_ORDER.index(name)
    n, k = LLAMA3_8B_SHAPES[name]
    w, _ = weights(n, k, seed=4000 + i)
    x, _ = activations(m, k, seed=2000 + i)
    return w, x


def small(n: int, k: int, m: int, seed: int, std: float = 0.02):
    """Small random case used by parity tests: W ~ N(0, std) with 0.1%..1 channel
    outliers x20 and X ~ N(0, 1)."""
    w, _ = weights(n, k, seed=seed, std=std, outlier_frac=max(1.0 / k, 0.001))
    x, _ = activations(m, k, seed=seed + 1)
    return w, x
