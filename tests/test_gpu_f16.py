"""GPU parity of the fused matmuls with fp16 activations and fp16 output
(gq_w4a16_gemv_f16 / _ws, gq_w4a16_gemm_f16 / _ws) against the oracle's
float64 group-by-group product of the same fp16 activations and exact
dequantized weight, to the matmul parity bar with the output's rounding taken
as half an fp16 ulp."""
import numpy as np
import pytest
import torch

from gpu_util import announce, device
from oracle import gq_oracle as O
from w4a16_dequant_gemm_group_amd import binding as B
import synth

pytestmark = pytest.mark.gpu


def _f16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(
        torch.float16).to(device())


def _weights(n, k, G, sym, seed):
    w, _ = synth.weights(n, k, seed=seed)
    codes, s, z = O.quantize_to_storage(w, 4, G, sym)
    return O.pack_int4(codes, sym), s, z


def _check(y, x_bits, qw, s, z, G, sym, what):
    x64 = O.f16_to_f64(x_bits)
    wh = O.dequantize_packed(qw, s, z, G, sym)
    ref = O.matmul_groupwise(x64, wh, G)
    yv = O.f16_to_f64(y.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    assert np.all(np.isfinite(yv)), what
    ok, rel, ratio = O.within_parity(yv, ref, x64, wh, out="f16")
    announce(f"{what}: relF={rel:.3e} max/allowed={ratio:.3f} (fp16 half-ulp bar)")
    assert ok, (what, rel, ratio)


@pytest.mark.parametrize("M,N,K,G,sym", [
    (1, 203, 6144, 128, False),
    (1, 4096, 14336, 32, True),
    (1, 130, 6400, 64, False),     # K not a multiple of 2048: per-lane offset tables
    (1, 1, 2048, 2048, True),
    (1, 77, 6144, 64, False),      # two lanes per group
    (1, 203, 4096, 64, True),
    (1, 9001, 2048, 256, False),   # several items per wave
    (2, 203, 6144, 128, False),    # streaming kernel, M activation rows
    (3, 203, 4096, 32, True),
    (4, 4096, 14336, 32, True),    # one 8-wave workgroup per compute unit
    (4, 16387, 4096, 128, False),  # four weight rows per item
    (5, 203, 4096, 64, False),     # matrix-core streaming kernel
    (8, 4096, 14336, 128, False),  # x streamed per item
    (12, 3001, 4096, 256, True),
    (16, 203, 4096, 32, True),
])
def test_gemv_f16(M, N, K, G, sym):
    qw, s, z = _weights(N, K, G, sym, seed=N + K)
    x, _ = synth.activations_f16(M, K, seed=K + M, n_outlier_channels=2)
    y = B.gq_w4a16_gemv_f16(_f16_dev(x), torch.from_numpy(qw).to(device()), _f16_dev(s),
                            None if sym else _f16_dev(z), G, sym)
    torch.cuda.synchronize()
    assert y.dtype == torch.float16 and y.shape == (M, N)
    _check(y, x, qw, s, None if sym else z, G, sym, f"gemv f16 M={M} [{N},{K}] G={G} sym={sym}")


@pytest.mark.parametrize("M,N,K,G,sym", [
    (300, 260, 640, 128, False),     # ragged, split K
    (2048, 512, 4096, 128, False),
    (96, 300, 1216, 64, True),       # odd number of k tiles
    (257, 131, 512, 512, False),
])
def test_gemm_f16(M, N, K, G, sym):
    qw, s, z = _weights(N, K, G, sym, seed=M + N)
    x, _ = synth.activations_f16(M, K, seed=M, n_outlier_channels=4)
    y = B.gq_w4a16_gemm_f16(_f16_dev(x), torch.from_numpy(qw).to(device()), _f16_dev(s),
                            None if sym else _f16_dev(z), G, sym)
    torch.cuda.synchronize()
    assert y.dtype == torch.float16
    _check(y, x, qw, s, None if sym else z, G, sym, f"gemm f16 M={M} [{N},{K}] G={G} sym={sym}")


@pytest.mark.parametrize("M,K,G,ws", [
    (16, 2304, 128, True),      # split-K matrix-core kernel (workspace), 16 rows
    (9, 3328, 128, True),       # K at most 4096, not a multiple of 512
    (16, 2304, 32, True),       # group 32 through the split kernel
    (9, 3328, 128, False),      # no workspace: the per-row dot-product kernel
    (6, 4160, 64, False),
    (12, 14336, 32, False),     # long K: x streamed per item (no workspace needed)
    (7, 4352, 128, False),
])
def test_gemv_f16_split_and_dot_product_shapes(M, K, G, ws):
    qw, s, z = _weights(203, K, G, False, seed=M + K)
    x, _ = synth.activations_f16(M, K, seed=K - M, n_outlier_channels=2)
    args = (_f16_dev(x), torch.from_numpy(qw).to(device()), _f16_dev(s), _f16_dev(z), G, False)
    need = B.gq_w4a16_gemv_workspace_size(M, K, 203, G)
    if ws:
        assert need > 0
        y = B.gq_w4a16_gemv_f16(*args)
    else:
        y = B.gq_w4a16_plain("gq_w4a16_gemv_f16", *args)
    torch.cuda.synchronize()
    _check(y, x, qw, s, z, G, False, f"gemv f16 M={M} [203,{K}] G={G} workspace={ws and need > 0}")


@pytest.mark.parametrize("M,N,K,G,sym", [
    (300, 260, 4096, 32, False),   # group 32: the generic kernel
    (130, 200, 4128, 96, True),    # K % 64 == 32, group 96
])
def test_gemm_f16_generic_kernel(M, N, K, G, sym):
    qw, s, z = _weights(N, K, G, sym, seed=M + K)
    x, _ = synth.activations_f16(M, K, seed=M, n_outlier_channels=4)
    y = B.gq_w4a16_gemm_f16(_f16_dev(x), torch.from_numpy(qw).to(device()), _f16_dev(s),
                            None if sym else _f16_dev(z), G, sym)
    torch.cuda.synchronize()
    _check(y, x, qw, s, None if sym else z, G, sym, f"gemm f16 generic M={M} [{N},{K}] G={G}")
