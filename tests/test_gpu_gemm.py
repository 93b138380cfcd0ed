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
import synth

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


@pytest.mark.parametrize("M,N,K,G,sym", [
    (1000, 12288, 1024, 128, False),   # 4 x 48 = 192 tiles of 256 columns -> 256 of 192
    (1024, 12288, 1536, 64, True),     # the same with whole row tiles, symmetric g64
])
def test_192_column_tiles(M, N, K, G, sym):
    """Where 256-wide tiles would leave part of the GPU idle without a split
    and 192-wide ones fill it exactly, the 256-row kernel runs 256 x 192 tiles
    (waves of 64 x 96): every output against the oracle, ragged M."""
    w, _ = synth.weights(N, K, seed=N + K + G)
    x, _ = synth.activations(M, K, seed=M + 3, n_outlier_channels=4)
    qw, s, z = _oracle_weights(w, G, sym)
    y = B.gq_w4a16_gemm(bf16_dev(x), u8_dev(qw), f16_dev(s), None if sym else f16_dev(z), G, sym)
    torch.cuda.synchronize()
    ref = O.w4a16_reference(x, qw, s, z, G, sym)
    wh = O.dequantize_packed(qw, s, z, G, sym)
    assert_parity(bits16(y), ref, O.bf16_to_f64(x), wh, f"gemm [{M}x{N}x{K}] G={G} sym={sym} (192-wide tiles)")


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


def _split_case(M, N, K, G, sym, seed):
    w, _ = synth.weights(N, K, seed=seed)
    x, _ = synth.activations(M, K, seed=seed + 1, n_outlier_channels=4)
    qw, s, z = _oracle_weights(w, G, sym)
    z = None if sym else z
    dev = (bf16_dev(x), u8_dev(qw), f16_dev(s), None if sym else f16_dev(z))
    ref = O.w4a16_reference(x, qw, s, z, G, sym)
    wh = O.dequantize_packed(qw, s, z, G, sym)
    return x, dev, ref, wh


def test_split_workspace_with_stale_content():
    """The split GEMM takes caller memory of any content: a workspace filled
    with random bytes, then reused by a split of falling and then rising tile
    counts (handshake words of one call overlapping partial sums of another),
    gives oracle parity each time and bit-equal repeats."""
    announce("gemm split with a stale caller workspace: 128, 4, then 64 split tiles")
    K, G = 2048, 128
    need = max(B.gq_w4a16_gemm_workspace_size(512, K, n, G) for n in (64 * 256, 2 * 256, 32 * 256))
    assert need > 0
    g = torch.Generator(device="cuda").manual_seed(5)
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda", generator=g)
    for n, seed in ((64 * 256, 31), (2 * 256, 37), (32 * 256, 41)):
        x, (xd, qd, sd, zd), ref, wh = _split_case(512, n, K, G, False, seed)
        y = B.gq_w4a16_gemm(xd, qd, sd, zd, G, False, workspace=ws)
        y2 = B.gq_w4a16_gemm(xd, qd, sd, zd, G, False, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y, y2)
        cols = np.sort(np.random.default_rng(seed).choice(n, 96, replace=False))
        assert_parity(bits16(y)[:, cols], ref[:, cols], O.bf16_to_f64(x), wh,
                      f"split [{n},{K}] M=512, stale workspace, sampled columns")


@pytest.mark.parametrize("name", ["gq_w4a16_gemm", "gq_w4a16_gemm_f16"])
def test_plain_entry_point_runs_unsplit(name):
    """gq_w4a16_gemm without a workspace computes every tile in one workgroup;
    its result meets parity like the split one."""
    M, N, K, G = 512, 512, 2048, 128
    assert B.gq_w4a16_gemm_workspace_size(M, K, N, G) > 0       # a split is available
    w, _ = synth.weights(N, K, seed=71)
    qw, s, z = _oracle_weights(w, G, False)
    wh = O.dequantize_packed(qw, s, z, G, False)
    if name.endswith("_f16"):
        x, _ = synth.activations_f16(M, K, seed=72, n_outlier_channels=4)
        x64 = O.f16_to_f64(x)
        y = B.gq_w4a16_plain(name, f16_dev(x), u8_dev(qw), f16_dev(s), f16_dev(z), G, False)
        torch.cuda.synchronize()
        ok, rel, ratio = O.within_parity(O.f16_to_f64(bits16(y)), O.matmul_groupwise(x64, wh, G),
                                         x64, wh, out="f16")
        announce(f"{name} unsplit: relF={rel:.3e} max/allowed={ratio:.3f}")
        assert ok
        return
    x, _ = synth.activations(M, K, seed=72, n_outlier_channels=4)
    y = B.gq_w4a16_plain(name, bf16_dev(x), u8_dev(qw), f16_dev(s), f16_dev(z), G, False)
    torch.cuda.synchronize()
    assert_parity(bits16(y), O.w4a16_reference(x, qw, s, z, G, False), O.bf16_to_f64(x), wh,
                  f"{name} unsplit [{N},{K}] M={M}")


def test_split_timeout_poisons_the_tile(monkeypatch):
    """Forced from the host: with the handshake's poll bound set to 0 the
    second half of every split tile gives up at once and writes NaN over its
    tile instead of a partial sum (every workgroup exits normally).  With the
    bound restored the same call is exact again."""
    M, N, K, G = 512, 512, 2048, 128
    announce("gemm split handshake, poll bound 0 (host-forced timeout)")
    x, (xd, qd, sd, zd), ref, wh = _split_case(M, N, K, G, False, 81)
    ws = torch.zeros(B.gq_w4a16_gemm_workspace_size(M, K, N, G), dtype=torch.uint8, device="cuda")
    monkeypatch.setenv("GQ_SPLIT_POLL_LIMIT", "0")
    y = B.gq_w4a16_gemm(xd, qd, sd, zd, G, False, workspace=ws)
    torch.cuda.synchronize()
    monkeypatch.delenv("GQ_SPLIT_POLL_LIMIT")
    yf = y.float().cpu().numpy()
    # four split tiles of 256 x 256: each is either all NaN (its second half
    # timed out) or never written by a NaN
    tiles = [yf[i:i + 256, j:j + 256] for i in (0, 256) for j in (0, 256)]
    assert all(np.isnan(t).all() or not np.isnan(t).any() for t in tiles)
    assert sum(np.isnan(t).all() for t in tiles) == 4
    y2 = B.gq_w4a16_gemm(xd, qd, sd, zd, G, False, workspace=ws)
    torch.cuda.synchronize()
    assert_parity(bits16(y2), ref, O.bf16_to_f64(x), wh, "split after a forced timeout")


@pytest.mark.parametrize("M,N,K,G,sym", [
    (512, 512, 2048, 128, False),    # 4 tiles: K split in two halves of 16 tiles
    (300, 700, 1216, 64, True),      # ragged, odd number of 64-k tiles, symmetric
    (256, 256, 2560, 256, False),    # one tile, split on a 256-group boundary
])
def test_split_k_and_graph_capture(M, N, K, G, sym):
    """Grids that fill at most half the GPU split K in two; both halves must
    agree with the oracle.  Under graph capture the binding takes the workspace
    from the graph's pool, so the captured GEMM runs split as well; every replay
    (with eager work between them) reproduces the eager result bit for bit."""
    announce(f"gemm split-K M={M} N={N} K={K} G={G} sym={sym}")
    assert B.gq_w4a16_gemm_workspace_size(M, K, N, G, sym) > 0
    x, (xd, qd, sd, zd), ref, wh = _split_case(M, N, K, G, sym, K + 3)
    y_eager = B.gq_w4a16_gemm(xd, qd, sd, zd, G, sym)
    y_again = B.gq_w4a16_gemm(xd, qd, sd, zd, G, sym)
    torch.cuda.synchronize()
    assert torch.equal(y_eager, y_again)  # the two-term combine does not depend on timing
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
    for rep in range(3):
        y_g.zero_()
        g.replay()
        B.gq_w4a16_gemm(xd[:64], qd, sd, zd, G, sym)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_eager), f"replay {rep}"
