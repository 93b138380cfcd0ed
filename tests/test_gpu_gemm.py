"""GPU parity of the fused W4A16 MFMA GEMM against the oracle's float64 product.

Small cases span several 256x128 output tiles, ragged M/N/K tails and every
group size path (32, 64, 96, 128, K); the Llama-3-8B prefill shapes
(M = 2048, asym g128, activations with 4 channels x50) run at full size in the
bench's launch configuration and are checked on sampled rows and columns.
"""
import numpy as np
import pytest
import torch

from gpu_util import announce, assert_parity, bf16_dev, bits16, f16_dev, u8_dev
from oracle import gq_oracle as O
from w4a16_dequant_gemm_group_amd import binding as B
from w4a16_dequant_gemm_group_amd import synth

pytestmark = pytest.mark.gpu


def _oracle_weights(w_bits, G, sym):
    codes, s_bits, z_bits = O.quantize_to_storage(w_bits, 4, G, sym)
    return O.pack_int4(codes, sym), s_bits, z_bits


@pytest.mark.parametrize("M,N,K,G,sym", [
    (256, 128, 128, 128, False),     # exactly one tile
    (300, 260, 640, 128, False),     # ragged M and N, 10 k tiles
    (64, 384, 1024, 32, True),       # small M, group 32 (two groups per k tile)
    (513, 200, 4096, 64, False),
    (100, 128, 96, 96, False),       # K = 96 = one group, half a k tile
    (2, 70, 864, 96, True),          # groups straddle k tiles
    (257, 131, 512, 512, False),     # group = K
    (1, 128, 256, 32, False),        # M = 1 through the GEMM
    # 256 x 256 tile kernel (K % 64 == 0, G in 64, 128, 256k)
    (260, 300, 832, 64, True),       # symmetric, odd number of k tiles
    (640, 64, 1216, 64, False),      # 19 k tiles, N below one tile
    (384, 520, 2560, 256, False),    # ten 256-groups, ragged N
    (512, 256, 1792, 256, True),     # symmetric, seven 256-groups
    (300, 1000, 1536, 128, True),    # symmetric g128, ragged M and N
])
def test_small_shapes(M, N, K, G, sym):
    w, _ = synth.weights(N, K, seed=N + K)
    x, _ = synth.activations(M, K, seed=M + 1, n_outlier_channels=min(4, K // 32))
    qw, s, z = _oracle_weights(w, G, sym)
    y = B.gq_w4a16_gemm(bf16_dev(x), u8_dev(qw), f16_dev(s), None if sym else f16_dev(z), G, sym)
    torch.cuda.synchronize()
    ref = O.w4a16_reference(x, qw, s, z, G, sym)
    wh = O.dequantize_packed(qw, s, z, G, sym)
    assert_parity(bits16(y), ref, O.bf16_to_f64(x), wh, f"gemm [{M}x{N}x{K}] G={G} sym={sym}")


def test_matches_gemv_on_small_m():
    """For M <= 16 the GEMM and GEMV compute the same product."""
    w, x = synth.small(256, 4096, 8, seed=12)
    qw, s, z = _oracle_weights(w, 128, False)
    args = (u8_dev(qw), f16_dev(s), f16_dev(z), 128, False)
    yg = O.bf16_to_f64(bits16(B.gq_w4a16_gemm(bf16_dev(x), *args)))
    yv = O.bf16_to_f64(bits16(B.gq_w4a16_gemv(bf16_dev(x), *args)))
    assert O.rel_frobenius(yg, yv) < 3e-3


@pytest.mark.parametrize("name", synth.SHAPE_ORDER)
def test_prefill_shapes_full_size(name):
    w, x = synth.prefill_case(name)
    codes, scales, zeros = B.gq_quantize_groups(bf16_dev(w), 4, 128, False)
    qw = B.gq_pack_int4(codes)
    y = B.gq_w4a16_gemm(bf16_dev(x), qw, scales, zeros, 128, False)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    rows = np.sort(rng.choice(w.shape[0], 192, replace=False))
    ms = np.sort(rng.choice(x.shape[0], 96, replace=False))
    qw_ref, s_ref, z_ref = _oracle_weights(w[rows], 128, False)
    assert np.array_equal(qw.cpu().numpy()[rows], qw_ref)
    ref = O.w4a16_reference(x[ms], qw_ref, s_ref, z_ref, 128, False)
    wh = O.dequantize_packed(qw_ref, s_ref, z_ref, 128, False)
    yb = bits16(y)[np.ix_(ms, rows)]
    # the max-error bound uses ||x||_inf of the whole activation
    assert_parity(yb, ref, O.bf16_to_f64(x), wh, f"gemm {name} M=2048 full, sampled")


@pytest.mark.parametrize("G", [32, 64, 128, 256])
def test_zero_scale_groups(G):
    """Groups whose fp16 scale is 0 contribute nothing (x^ = 0 * (q - z) = 0),
    including the first group of a column and runs of zero-scale groups; the
    GEMM's running-scale accumulation must skip them exactly."""
    M, N, K = 130, 260, 1024
    w, _ = synth.weights(N, K, seed=31)
    x, _ = synth.activations(M, K, seed=32, n_outlier_channels=4)
    qw, s, z = _oracle_weights(w, G, False)
    s = s.copy()
    s[0, :] = 0                     # a whole column of zero scales
    s[1, 0] = 0                     # the first group
    s[2, 1:4] = 0                   # a run in the middle
    s[3, -1] = 0                    # the last group
    s[5::7, 2] = 0                  # scattered
    y = B.gq_w4a16_gemm(bf16_dev(x), u8_dev(qw), f16_dev(s), f16_dev(z), G, False)
    yv = B.gq_w4a16_gemv(bf16_dev(x[:3]), u8_dev(qw), f16_dev(s), f16_dev(z), G, False)
    torch.cuda.synchronize()
    ref = O.w4a16_reference(x, qw, s, z, G, False)
    wh = O.dequantize_packed(qw, s, z, G, False)
    assert np.all(ref[:, 0] == 0.0)
    assert np.all(bits16(y)[:, 0] & 0x7FFF == 0)
    assert_parity(bits16(y), ref, O.bf16_to_f64(x), wh, f"gemm zero-scale groups G={G}")
    assert_parity(bits16(yv), ref[:3], O.bf16_to_f64(x[:3]), wh, f"gemv zero-scale groups G={G}")


def test_last_round_split():
    """300 output tiles on 256 compute units: 256 whole tiles, then the last
    44 tiles with K split in two (88 workgroups).  Columns sampled from both
    launches against the oracle; two calls agree bit for bit."""
    M, N, K, G = 256, 300 * 256, 1024, 128
    announce(f"gemm last-round split M={M} N={N} K={K} G={G}")
    w, _ = synth.weights(N, K, seed=17)
    x, _ = synth.activations(M, K, seed=19, n_outlier_channels=4)
    codes, scales, zeros = B.gq_quantize_groups(bf16_dev(w), 4, G, False)
    qw = B.gq_pack_int4(codes)
    xd = bf16_dev(x)
    y = B.gq_w4a16_gemm(xd, qw, scales, zeros, G, False)
    y2 = B.gq_w4a16_gemm(xd, qw, scales, zeros, G, False)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    rng = np.random.default_rng(23)
    cut = 256 * 256  # first column of the split launch (one 256-row M tile)
    rows = np.sort(np.concatenate([rng.choice(cut, 64, replace=False),
                                   cut + rng.choice(N - cut, 64, replace=False)]))
    qw_ref, s_ref, z_ref = _oracle_weights(w[rows], G, False)
    assert np.array_equal(qw.cpu().numpy()[rows], qw_ref)
    ref = O.w4a16_reference(x, qw_ref, s_ref, z_ref, G, False)
    wh = O.dequantize_packed(qw_ref, s_ref, z_ref, G, False)
    assert_parity(bits16(y)[:, rows], ref, O.bf16_to_f64(x), wh, f"last-round split [{N},{K}] M={M}")


def test_split_scratch_reuse():
    """Split GEMMs of falling then rising tile counts on one stream reuse the
    library scratch without reallocating it: the per-tile counters of the
    later, larger split must not overlap partial sums an earlier, smaller split
    left behind.  Checked against the oracle and for bit-equal repeats."""
    M, K, G = 512, 2048, 128
    announce("gemm split scratch reuse: 128, 4, then 64 split tiles")
    def run(n, seed):
        w, _ = synth.weights(n, K, seed=seed)
        x, _ = synth.activations(M, K, seed=seed + 1, n_outlier_channels=4)
        codes, scales, zeros = B.gq_quantize_groups(bf16_dev(w), 4, G, False)
        qw = B.gq_pack_int4(codes)
        args = (bf16_dev(x), qw, scales, zeros, G, False)
        return w, x, qw, args, B.gq_w4a16_gemm(*args)
    run(64 * 256, 31)   # 128 tiles: the largest scratch
    run(2 * 256, 37)    # 4 tiles: partial sums at the start of the buffer
    w, x, qw, args, y = run(32 * 256, 41)  # 64 tiles: counters span more words
    y2 = B.gq_w4a16_gemm(*args)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    rows = np.sort(np.random.default_rng(43).choice(w.shape[0], 96, replace=False))
    qw_ref, s_ref, z_ref = _oracle_weights(w[rows], G, False)
    assert np.array_equal(qw.cpu().numpy()[rows], qw_ref)
    ref = O.w4a16_reference(x, qw_ref, s_ref, z_ref, G, False)
    wh = O.dequantize_packed(qw_ref, s_ref, z_ref, G, False)
    assert_parity(bits16(y)[:, rows], ref, O.bf16_to_f64(x), wh, "split after smaller split, sampled")


@pytest.mark.parametrize("M,N,K,G,sym", [
    (512, 512, 2048, 128, False),    # 4 tiles: K split in two halves of 16 tiles
    (300, 700, 1216, 64, True),      # ragged, odd number of 64-k tiles, symmetric
    (256, 256, 2560, 256, False),    # one tile, split on a 256-group boundary
])
def test_split_k_and_graph_capture(M, N, K, G, sym):
    """Grids that fill at most half the GPU split K in two; both halves must
    agree with the oracle.  Under graph capture the library hands out no
    scratch, so the captured GEMM runs unsplit; every replay reproduces it."""
    announce(f"gemm split-K M={M} N={N} K={K} G={G} sym={sym}")
    w, _ = synth.weights(N, K, seed=K + 3)
    x, _ = synth.activations(M, K, seed=M + 5, n_outlier_channels=4)
    qw, s, z = _oracle_weights(w, G, sym)
    xd, qd, sd = bf16_dev(x), u8_dev(qw), f16_dev(s)
    zd = None if sym else f16_dev(z)
    y_eager = B.gq_w4a16_gemm(xd, qd, sd, zd, G, sym)
    y_again = B.gq_w4a16_gemm(xd, qd, sd, zd, G, sym)
    torch.cuda.synchronize()
    assert torch.equal(y_eager, y_again)  # the two-term combine does not depend on timing
    ref = O.w4a16_reference(x, qw, s, None if sym else z, G, sym)
    wh = O.dequantize_packed(qw, s, None if sym else z, G, sym)
    assert_parity(bits16(y_eager), ref, O.bf16_to_f64(x), wh, f"split-K [{N},{K}] M={M}")

    y_g = torch.empty_like(y_eager)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        B.gq_w4a16_gemm(xd, qd, sd, zd, G, sym, y=y_g)
        with torch.cuda.graph(g, stream=stream):
            B.gq_w4a16_gemm(xd, qd, sd, zd, G, sym, y=y_g)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    first = None
    for rep in range(3):
        y_g.zero_()
        g.replay()
        B.gq_w4a16_gemm(xd[:64], qd, sd, zd, G, sym)  # eager work between replays
        torch.cuda.synchronize()
        if first is None:
            first = y_g.clone()
            assert_parity(bits16(y_g), ref, O.bf16_to_f64(x), wh, f"captured [{N},{K}] M={M}")
        assert torch.equal(y_g, first), f"replay {rep}"
