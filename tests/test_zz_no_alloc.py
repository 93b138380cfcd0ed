"""gq_w4a16_gemm_noalloc (split scratch in the library's fixed device array,
no allocation by the call) against gq_w4a16_gemm_ws with a caller workspace:
two calls in a row, the second with a smaller problem, each bit-equal to the
workspace entry point's output and within the oracle's parity bar."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import announce, assert_parity, bf16_dev, bits16, f16_dev, u8_dev
from oracle import gq_oracle as O
from w4a16_dequant_gemm_group_amd import binding as B
import synth

pytestmark = pytest.mark.gpu


def _case(M, N, K, G, seed):
    w, _ = synth.weights(N, K, seed=seed)
    x, _ = synth.activations(M, K, seed=seed + 1, n_outlier_channels=4)
    codes, s, z = O.quantize_to_storage(w, 4, G, False)
    qw = O.pack_int4(codes, False)
    return x, qw, s, z


def _call(fn, x, qw, s, z, G, y, *ws):
    M, K = x.shape
    N = qw.shape[0]
    st = fn(ctypes.c_void_p(x.data_ptr()), M, K, ctypes.c_void_p(qw.data_ptr()),
            ctypes.c_void_p(s.data_ptr()), ctypes.c_void_p(z.data_ptr()), N, B.qparams(4, G, False),
            ctypes.c_void_p(y.data_ptr()), *ws,
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == B.GQ_OK, B.lib().gq_status_str(st).decode()


def test_noalloc_gemm_matches_workspace_gemm():
    L = B.lib()
    G = 128
    # o-shaped prefill (128 split tiles: the whole array), then a smaller split
    # (4 tiles) that finds the first call's partial sums and handshake words
    for M, N, K, seed in ((2048, 4096, 4096, 101), (512, 512, 2048, 103)):
        announce(f"gemm noalloc M={M} N={N} K={K} G={G}")
        need = B.gq_w4a16_gemm_workspace_size(M, K, N, G)
        assert 0 < need <= (32 << 20) + 4096   # GQ_NOALLOC_SCRATCH_BYTES
        x, qw, s, z = _case(M, N, K, G, seed)
        xd, qd, sd, zd = bf16_dev(x), u8_dev(qw), f16_dev(s), f16_dev(z)
        y_na = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        y_ws = torch.empty_like(y_na)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        _call(L.gq_w4a16_gemm_noalloc, xd, qd, sd, zd, G, y_na)
        _call(L.gq_w4a16_gemm_ws, xd, qd, sd, zd, G, y_ws, ctypes.c_void_p(ws.data_ptr()),
              ctypes.c_size_t(need))
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ws)
        cols = np.sort(np.random.default_rng(seed).choice(N, min(N, 192), replace=False))
        ref = O.w4a16_reference(x, qw[cols], s[cols], z[cols], G, False)
        wh = O.dequantize_packed(qw[cols], s[cols], z[cols], G, False)
        assert_parity(bits16(y_na)[:, cols], ref, O.bf16_to_f64(x), wh,
                      f"noalloc [{N},{K}] M={M}, sampled columns")
