"""GPU checks of the comparators the 4-bit kernels are measured against: the
plain bf16 GEMV (against the float64 product x w^T of the same bf16 inputs, to
the matmul parity bar) and the HBM stream-read probe.  Also the unfused path
"dequantize into a bf16 weight, then multiply" that the fused kernel replaces,
against the oracle's product."""
import numpy as np
import pytest
import torch

from gpu_util import announce, bf16_dev, bf16_out_to_f64, device
from oracle import gq_oracle as O
from w4a16_dequant_gemm_group_amd import binding as B
import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,N", [
    (1, 8, 1), (1, 520, 7), (2, 4096, 203), (3, 2056, 4096), (4, 6144, 65),
    (1, 14336, 4096), (2, 14336, 33), (4, 8192, 9),
])
def test_bf16_gemv_matches_float64_product(M, K, N):
    announce(f"bf16 gemv M={M} K={K} N={N}")
    w, _ = synth.weights(N, K, seed=700 + K % 97)
    x, _ = synth.activations(M, K, seed=800 + N % 89, n_outlier_channels=2)
    y = B.gq_bf16_gemv(bf16_dev(x), bf16_dev(w))
    torch.cuda.synchronize()
    x64, w64 = O.bf16_to_f64(x), O.bf16_to_f64(w)
    ok, rel, ratio = O.within_parity(bf16_out_to_f64(y), x64 @ w64.T, x64, w64)
    assert ok, (rel, ratio)


def test_bf16_gemv_rows_past_the_grid_and_empty():
    announce("bf16 gemv edge cases")
    # N not a multiple of the 8 rows a workgroup owns; the output past N is untouched
    w, x = synth.small(13, 1024, 1, seed=6)
    out = torch.full((1, 16), 7.0, dtype=torch.bfloat16, device=device())
    B.gq_bf16_gemv(bf16_dev(x), bf16_dev(w), y=out[:, :13])   # a view of the first 13 of 16 columns
    torch.cuda.synchronize()
    assert torch.all(out[0, 13:] == 7.0)
    x64, w64 = O.bf16_to_f64(x), O.bf16_to_f64(w)
    ok, rel, ratio = O.within_parity(bf16_out_to_f64(out[:, :13]), x64 @ w64.T, x64, w64)
    assert ok, (rel, ratio)
    # M = 0 is a no-op
    B.gq_bf16_gemv(torch.empty((0, 1024), dtype=torch.bfloat16, device=device()), bf16_dev(w))


def test_stream_read_runs_over_sizes():
    announce("stream read")
    sink = torch.zeros(1, dtype=torch.int32, device=device())
    for nbytes in (16, 48, 32768 + 16, 3 << 20):
        buf = torch.arange(nbytes // 4, dtype=torch.int32, device=device())
        B.gq_stream_read(buf, sink)
    torch.cuda.synchronize()
    # the fold is stored only when it equals one fixed constant
    assert int(sink.item()) in (0, 0x2545F491 - (1 << 32))


@pytest.mark.parametrize("M,sym,G", [(1, False, 128), (2, True, 32), (4, False, 64)])
def test_unfused_dequantize_then_bf16_gemv(M, sym, G):
    """The unfused comparator: gq_dequantize -> bf16 W^ in HBM -> gq_bf16_gemv.
    Rounding W^ to bf16 adds error the fused kernel does not have, so the bar
    here is the oracle product of the bf16-rounded W^ (what this path computes)."""
    announce(f"unfused M={M} sym={sym} G={G}")
    N, K = 203, 4096
    w, x = synth.small(N, K, M, seed=40 + M)
    codes, s, z = B.gq_quantize_groups(bf16_dev(w), 4, G, sym)
    qw = B.gq_pack_int4(codes, sym)
    w_hat = B.gq_dequantize(qw, s, z, G, sym, out_dtype=torch.bfloat16)
    y = B.gq_bf16_gemv(bf16_dev(x), w_hat)
    torch.cuda.synchronize()
    c_ref, s_ref, z_ref = O.quantize_to_storage(w, 4, G, sym)
    wh64 = O.dequantize_packed(O.pack_int4(c_ref, sym), s_ref, z_ref, G, sym)
    wh_b = O.bf16_to_f64(O.f32_exact_to_bf16_bits(wh64))
    x64 = O.bf16_to_f64(x)
    ok, rel, ratio = O.within_parity(bf16_out_to_f64(y), x64 @ wh_b.T, x64, wh_b)
    assert ok, (rel, ratio)


def test_issue_rate_probes():
    """The matrix-core / vector-ALU and LDS probes run and report plausible
    per-wave loop cycles: at least 16 cycles per MFMA of the loop, not fewer
    when vector work is added, and LDS reads below 256 bytes per clock."""
    announce("issue-rate probes")
    iters = 200
    base = B.gq_probe_mfma_valu(0, iters, 4).cpu().numpy()
    more = B.gq_probe_mfma_valu(128, iters, 4).cpu().numpy()
    assert np.all(base > 0) and np.all(more > 0)
    assert np.median(base) / iters >= 8 * 16
    assert np.median(more) >= np.median(base) * 0.95
    waves = 8
    lds = B.gq_probe_lds_read(waves, iters, 4).cpu().numpy().reshape(4, waves)
    bpc = waves * iters * 16 * 1024 / lds.max(axis=1)
    assert np.all(bpc > 8) and np.all(bpc < 256), bpc
