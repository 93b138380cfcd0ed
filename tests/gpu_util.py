"""Helpers for the GPU parity tests: device setup, host<->device copies of the
uint16 bit arrays, and the parity bar of the matmuls.

Parity bar (both must hold): relative Frobenius error <= 2e-3 and, per
element, |y - y_ref| <= 1e-2 * ||x||_inf * ||w^||_inf * sqrt(K) / 64 plus half a
bf16 ulp of the output, where y_ref is the oracle's float64 product and the
norms are element-wise maxima over the whole activation and dequantized weight.
"""
import sys

import numpy as np
import torch

from oracle import gq_oracle as O

REL_F = 2e-3


def device():
    return torch.device("cuda:0")


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bits -> bf16 tensor on the GPU."""
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(device())


def f16_dev(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.float16)
    return t.to(device())


def u8_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device())


def bits16(t: torch.Tensor) -> np.ndarray:
    """bf16/fp16 tensor -> uint16 bit array on the host."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_out_to_f64(t: torch.Tensor) -> np.ndarray:
    return O.bf16_to_f64(bits16(t))


def assert_parity(y_bits: np.ndarray, y_ref: np.ndarray, x64: np.ndarray, w_hat: np.ndarray, what: str):
    y = O.bf16_to_f64(y_bits)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    ok, rel, ratio = O.within_parity(y, y_ref, x64, w_hat)
    mx = float(np.abs(y - y_ref).max())
    announce(f"{what}: relF={rel:.3e} (<= {REL_F}), max={mx:.3e}, "
             f"max/allowed={ratio:.3f} (<= 1; bound {O.max_err_bound(x64, w_hat):.3e} + half bf16 ulp)")
    assert rel <= REL_F, f"{what}: relative Frobenius error {rel:.3e} > {REL_F}"
    assert ratio <= 1.0, f"{what}: element error exceeds the bound by x{ratio:.3f}"
    return rel, mx
