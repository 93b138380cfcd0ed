"""GPU parity of the fused W4A16 GEMV against the oracle's float64 product.

Packed weights come from the oracle (so the GEMV is tested on its own); one
test runs the whole GPU path (quantize -> pack -> GEMV) end to end.  Sizes span
several 2048-wide k steps, ragged k tails, row counts that are not a multiple
of the rows per workgroup, every M the kernel instantiates, both schemes and
several group sizes; the Llama-3-8B decode shapes run at full size with the
bench's launch configuration and are checked on sampled rows.
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
    qw = O.pack_int4(codes, sym)
    return qw, s_bits, z_bits


def _run(x_bits, qw, s_bits, z_bits, G, sym, what, rows=None):
    x = bf16_dev(x_bits)
    y = B.gq_w4a16_gemv(x, u8_dev(qw), f16_dev(s_bits), None if sym else f16_dev(z_bits), G, sym)
    torch.cuda.synchronize()
    yb = bits16(y)
    r = slice(None) if rows is None else rows
    ref = O.w4a16_reference(x_bits, qw[r], s_bits[r], None if sym else z_bits[r], G, sym)
    wh = O.dequantize_packed(qw[r], s_bits[r], None if sym else z_bits[r], G, sym)
    return assert_parity(yb[:, r], ref, O.bf16_to_f64(x_bits), wh, what)


@pytest.mark.parametrize("G", [128, 512])
def test_tiny_reference(G):
    w, x = synth.tiny_reference()
    qw, s, z = _oracle_weights(w, G, False)
    _run(x, qw, s, z, G, False, f"tiny [256,512] M=1 asym G={G}")


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 11, 16])
@pytest.mark.parametrize("sym,G", [(False, 128), (True, 32), (False, 64), (True, 96)])
def test_small_shapes(M, sym, G):
    # K = 6144 + 384: three full 2048 steps plus a ragged tail; N = 203 rows
    K = 6528 if G != 96 else 6528 - 6528 % 96
    w, x = synth.small(203, K, M, seed=M * 7 + G)
    qw, s, z = _oracle_weights(w, G, sym)
    _run(x, qw, s, z, G, sym, f"[203,{K}] M={M} sym={sym} G={G}")


@pytest.mark.parametrize("M", [4, 5, 8, 9, 16])
@pytest.mark.parametrize("sym,G", [(True, 32), (False, 64), (False, 128), (False, 256), (True, 512)])
def test_small_batch_matrix_core_shapes(M, sym, G):
    # the split-K matrix-core path (4 <= M <= 16, K % 256 == 0): K ends inside
    # a 1024-wide slice and N = 203 leaves a partial 64-row group
    K = 6656 if G == 512 else 6400
    w, x = synth.small(203, K, M, seed=M * 13 + G)
    qw, s, z = _oracle_weights(w, G, sym)
    _run(x, qw, s, z, G, sym, f"[203,{K}] M={M} sym={sym} G={G} (matrix cores)")


@pytest.mark.parametrize("K", [32, 96, 2048, 2080, 16384, 18432, 40960, 65536, 67584])
def test_k_extents(K):
    # one lane's worth of k up to more than one LDS chunk (8 steps) of k; at
    # M = 1 the streaming kernel stages x in several passes up to K = 65536
    # (32 steps) and the per-row kernel takes 67584
    w, x = synth.small(67, K, 1, seed=K)
    G = 32 if K % 128 else 128
    qw, s, z = _oracle_weights(w, G, False)
    _run(x, qw, s, z, G, False, f"[67,{K}] M=1 G={G}")


@pytest.mark.parametrize("sym,G", [(False, 32), (True, 32), (False, 64), (True, 64), (False, 128),
                                   (True, 128), (False, 256), (True, 512), (False, 1024),
                                   (False, 2048)])
@pytest.mark.parametrize("N,K", [(203, 6144), (9001, 2048)])
def test_m1_stream_group_sizes(N, K, sym, G):
    # M = 1 with K a multiple of 2048 (fixed per-lane offsets) for every group
    # size that divides 2048: one to 64 lanes per group.  N is odd (the last
    # row pair has one real row); N = 9001 gives every wave several items.
    w, x = synth.small(N, K, 1, seed=N + G + sym)
    qw, s, z = _oracle_weights(w, G, sym)
    rows = None if N < 1000 else np.r_[0:64, N - 64:N]
    _run(x, qw, s, z, G, sym, f"[{N},{K}] M=1 sym={sym} G={G} (stream)", rows=rows)


@pytest.mark.parametrize("M", [2, 3, 4])
@pytest.mark.parametrize("N,K,sym,G", [
    (16387, 4096, False, 128),   # enough items for four weight rows per item (M >= 3)
    (203, 10240, True, 32),      # x needs one workgroup of 8 waves per compute unit (M >= 3)
    (203, 10368, False, 128),    # the same with per-lane offset tables (K % 2048 != 0)
])
def test_stream_multi_row_layouts(M, N, K, sym, G):
    w, x = synth.small(N, K, M, seed=N + K + M)
    qw, s, z = _oracle_weights(w, G, sym)
    rows = None if N < 1000 else np.r_[0:64, N // 2:N // 2 + 64, N - 67:N]
    _run(x, qw, s, z, G, sym, f"[{N},{K}] M={M} sym={sym} G={G} (stream, M > 1)", rows=rows)


@pytest.mark.parametrize("M", [5, 8, 9, 16])
@pytest.mark.parametrize("N,K,sym,G", [
    (203, 4096, True, 32), (203, 4096, False, 64), (203, 4096, False, 128),
    (203, 4096, True, 256), (203, 4096, False, 512), (203, 4096, True, 1024),
    (16387, 4096, False, 128),   # several row blocks per workgroup
    # M > 8: two teams of 8 waves per workgroup (>= 2 row blocks per compute
    # unit; 1025 row blocks: the last workgroup's second team runs empty items)
    (16387, 4096, True, 32), (16387, 4096, False, 32),
])
def test_mfma_stream_shapes(M, N, K, sym, G):
    # the matrix-core GEMV with every activation row in LDS and K split over a
    # workgroup's waves (no scratch): all group classes, a partial last row
    # block, rows beyond M dropped
    assert B.gq_w4a16_gemv_workspace_size(M, K, N, G, sym) == 0
    w, x = synth.small(N, K, M, seed=N + K + M + G)
    qw, s, z = _oracle_weights(w, G, sym)
    rows = None if N < 1000 else np.r_[0:64, N // 2:N // 2 + 64, N - 67:N]
    _run(x, qw, s, z, G, sym, f"[{N},{K}] M={M} sym={sym} G={G} (matrix cores, streaming)", rows=rows)


@pytest.mark.parametrize("M", [4, 5, 8, 13])
@pytest.mark.parametrize("K", [1024, 2048, 6144, 8192, 14336, 16896, 18432])
def test_mfma_stream_k_extents(M, K):
    # (M = 4 and M > 4 take the register-x kernel at K = 1024 and 2048; beyond
    # 4096 M = 4 takes the dot-product streaming kernel and M > 4 the
    # streamed-x kernel; none of them with scratch)
    assert B.gq_w4a16_gemv_workspace_size(M, K, 333, 64, False) == 0
    w, x = synth.small(333, K, M, seed=M + K)
    qw, s, z = _oracle_weights(w, 64, False)
    _run(x, qw, s, z, 64, False, f"[333,{K}] M={M} asym G=64 (matrix cores, streaming)")


def test_group_equals_k_and_outlier_blowup():
    """Per-row (group = K) quantization of the outlier case loses far more
    accuracy than group 128 (S08 page, outlier remarks); both GPU results are
    still within the parity bar of their own oracle."""
    w, x = synth.tiny_reference()
    errs = {}
    for G in (128, 512):
        qw, s, z = _oracle_weights(w, G, False)
        y = B.gq_w4a16_gemv(bf16_dev(x), u8_dev(qw), f16_dev(s), f16_dev(z), G, False)
        exact = O.bf16_to_f64(x) @ O.bf16_to_f64(w).T
        errs[G] = O.rel_frobenius(O.bf16_to_f64(bits16(y)), exact)
    announce(f"error vs unquantized product: G=128 {errs[128]:.3e}, G=512 {errs[512]:.3e}")
    assert errs[512] > 1.5 * errs[128]


def full_rows_parity(y_bits, w, x, qw_dev, G, sym, what, chunk=4096):
    """Every output row against the oracle: the weight is quantized by the
    oracle in row chunks (bytes compared with the GPU's packed weight), the
    float64 product computed chunk by chunk, and the parity bar applied to the
    whole output with the whole dequantized weight's max |w^|."""
    N = w.shape[0]
    ref = np.empty((x.shape[0], N))
    wmax = 0.0
    qw_all = qw_dev.cpu().numpy()
    for r0 in range(0, N, chunk):
        r1 = min(N, r0 + chunk)
        qw_ref, s_ref, z_ref = _oracle_weights(w[r0:r1], G, sym)
        assert np.array_equal(qw_all[r0:r1], qw_ref), (what, r0)
        wh = O.dequantize_packed(qw_ref, s_ref, z_ref, G, sym)
        wmax = max(wmax, float(np.abs(wh).max()))
        ref[:, r0:r1] = O.matmul_groupwise(O.bf16_to_f64(x), wh, G)
    assert_parity(y_bits, ref, O.bf16_to_f64(x), np.array([[wmax]]), what)


@pytest.mark.parametrize("name", synth.SHAPE_ORDER)
def test_decode_shapes_full_size(name):
    """Llama-3-8B decode GEMV at full size (M=1, asym g128), in the bench's
    launch configuration: every output row against the oracle."""
    w, x = synth.decode_case(name)
    announce(f"decode {name} {w.shape} M=1, all rows")
    codes, scales, zeros = B.gq_quantize_groups(bf16_dev(w), 4, 128, False)
    qw = B.gq_pack_int4(codes)
    del codes
    y = B.gq_w4a16_gemv(bf16_dev(x), qw, scales, zeros, 128, False)
    torch.cuda.synchronize()
    full_rows_parity(bits16(y), w, x, qw, 128, False, f"{name} {w.shape} M=1 full, all rows")


@pytest.mark.parametrize("name,M", [("down", 2), ("down", 4), ("down", 8), ("down", 16),
                                    ("gate_up", 2), ("gate_up", 3), ("gate_up", 4), ("qkv", 4),
                                    ("gate_up", 8), ("gate_up", 16), ("o", 12)])
def test_small_batch_full_size_sym_g32(name, M):
    # M <= 3 take the dot-product streaming kernel, M >= 4 at K = 4096 the
    # register-x matrix-core kernel, M = 2..4 on down the dot-product kernel
    # and M > 4 there the streamed-x one
    w, _ = synth.decode_case(name)
    x, _ = synth.activations(M, w.shape[1], seed=2003)
    rows = np.sort(np.random.default_rng(4).choice(w.shape[0], 256, replace=False))
    codes, scales, _ = B.gq_quantize_groups(bf16_dev(w), 4, 32, True)
    qw = B.gq_pack_int4(codes, True)
    y = B.gq_w4a16_gemv(bf16_dev(x), qw, scales, None, 32, True)
    torch.cuda.synchronize()
    qw_ref, s_ref, _ = _oracle_weights(w[rows], 32, True)
    ref = O.w4a16_reference(x, qw_ref, s_ref, None, 32, True)
    wh = O.dequantize_packed(qw_ref, s_ref, None, 32, True)
    assert_parity(bits16(y)[:, rows], ref, O.bf16_to_f64(x), wh, f"{name} M={M} sym g32 full, sampled")


def test_special_inputs():
    """One-hot activation selects a dequantized column; zero activation gives 0."""
    w, _ = synth.small(64, 4096, 1, seed=5)
    qw, s, z = _oracle_weights(w, 128, False)
    wh = O.dequantize_packed(qw, s, z, 128, False)
    for k in (0, 1, 2047, 2048, 4095):
        e = np.zeros((1, 4096), np.float32); e[0, k] = 1.0
        xb = synth.f32_to_bf16_bits(e)
        y = B.gq_w4a16_gemv(bf16_dev(xb), u8_dev(qw), f16_dev(s), f16_dev(z), 128, False)
        want = O.f32_exact_to_bf16_bits(wh[:, k])
        assert np.array_equal(bits16(y)[0], want), k
    xz = np.zeros((2, 4096), np.uint16)
    y = B.gq_w4a16_gemv(bf16_dev(xz), u8_dev(qw), f16_dev(s), f16_dev(z), 128, False)
    assert np.all(bits16(y) & 0x7FFF == 0)


def test_misaligned_pointer_rejected():
    w, x = synth.small(16, 256, 1, seed=1)
    qw, s, z = _oracle_weights(w, 128, False)
    xd = torch.empty(4096 + 8, dtype=torch.bfloat16, device="cuda:0")[1:257].view(1, 256)
    with pytest.raises(B.GqError) as e:
        B.gq_w4a16_gemv(xd, u8_dev(qw), f16_dev(s), f16_dev(z), 128, False)
    assert e.value.status == B.GQ_ERR_MISALIGNED


def test_split_slices_and_plain_entry_point():
    """Shapes that only the split-K matrix-core kernel takes fast: with a
    workspace (the binding's default) repeated calls of falling and rising N
    and M agree bit for bit; gq_w4a16_gemv without a workspace runs the per-row
    dot-product kernel.  Both meet the oracle on sampled rows."""
    K, G = 2304, 128  # at most 4096, not a multiple of 512: the split-K matrix-core path
    for M, N, seed in ((8, 3000, 90), (5, 64, 91), (16, 1000, 92), (8, 20000, 94), (8, 3000, 93)):
        announce(f"small-batch split slices M={M} N={N} K={K}")
        w, x = synth.small(N, K, M, seed=seed)
        codes, sd, zd = B.gq_quantize_groups(bf16_dev(w), 4, G, False)
        qd = B.gq_pack_int4(codes)
        xd = bf16_dev(x)
        assert B.gq_w4a16_gemv_workspace_size(M, K, N, G, False) > 0
        y_ws = B.gq_w4a16_gemv(xd, qd, sd, zd, G, False)
        y_ws2 = B.gq_w4a16_gemv(xd, qd, sd, zd, G, False)
        y_plain = B.gq_w4a16_plain("gq_w4a16_gemv", xd, qd, sd, zd, G, False)
        torch.cuda.synchronize()
        assert torch.equal(y_ws, y_ws2)
        rows = np.sort(np.random.default_rng(seed).choice(N, min(N, 256), replace=False))
        qw, s, z = _oracle_weights(w[rows], G, False)
        assert np.array_equal(qd.cpu().numpy()[rows], qw)
        ref = O.w4a16_reference(x, qw, s, z, G, False)
        wh = O.dequantize_packed(qw, s, z, G, False)
        assert_parity(bits16(y_ws)[:, rows], ref, O.bf16_to_f64(x), wh,
                      f"[{N},{K}] M={M} split slices, sampled")
        assert_parity(bits16(y_plain)[:, rows], ref, O.bf16_to_f64(x), wh,
                      f"[{N},{K}] M={M} no workspace (dot products), sampled")


def test_workspace_entry_point_and_graph_replays():
    # gq_w4a16_gemv_ws with a caller's buffer and with one the binding takes
    # from torch run the same kernels: identical bits.  Captured into a graph,
    # the call gets its scratch from the graph's pool and every replay must
    # reproduce the eager result, with other eager work on the stream between
    # replays.  (K = 2304, at most 4096 and not a multiple of 512, keeps the
    # call on the split-K matrix-core path.)
    M, K, N, G = 12, 2304, 1000, 32
    w, x = synth.small(N, K, M, seed=77)
    qw, s, _ = _oracle_weights(w, G, True)
    xd, qd, sd = bf16_dev(x), u8_dev(qw), f16_dev(s)
    need = B.gq_w4a16_gemv_workspace_size(M, K, N, G, True)
    assert need == 3 * M * N * 4
    y_auto = B.gq_w4a16_gemv(xd, qd, sd, None, G, True)
    ws = torch.full((need + 64,), 0xA5, dtype=torch.uint8, device=xd.device)
    y_ws = B.gq_w4a16_gemv(xd, qd, sd, None, G, True, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y_auto, y_ws)
    ref = O.w4a16_reference(x, qw, s, None, G, True)
    wh = O.dequantize_packed(qw, s, None, G, True)
    assert_parity(bits16(y_ws), ref, O.bf16_to_f64(x), wh, f"[{N},{K}] M={M} sym g32 via workspace")
    with pytest.raises(ValueError):
        B.gq_w4a16_gemv(xd, qd, sd, None, G, True, workspace=ws[:need - 16])

    y_g = torch.empty_like(y_auto)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        B.gq_w4a16_gemv(xd, qd, sd, None, G, True, y=y_g)  # warm-up on the capture stream
        with torch.cuda.graph(g, stream=stream):
            B.gq_w4a16_gemv(xd, qd, sd, None, G, True, y=y_g)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for rep in range(4):
        y_g.zero_()
        g.replay()
        other = B.gq_w4a16_gemv(xd[:5], qd, sd, None, G, True)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_auto), f"replay {rep}"
        assert other.shape == (5, N)


@pytest.mark.parametrize("M,K,N,G,sym", [
    (3, 4096, 1000, 32, True),      # streaming kernel, three activation rows
    (8, 4096, 1000, 128, False),    # matrix-core streaming kernel
    (8, 14336, 500, 64, False),     # the same with x staged in chunks
    (16, 4096, 700, 32, True),
])
def test_scratch_free_paths_under_graph_capture(M, K, N, G, sym):
    # these calls need no workspace, so a captured graph holds only the
    # kernel launch; every replay must reproduce the eager bits, with other
    # eager work on the stream between replays
    assert B.gq_w4a16_gemv_workspace_size(M, K, N, G, sym) == 0
    w, x = synth.small(N, K, M, seed=M + K + N)
    qw, s, z = _oracle_weights(w, G, sym)
    xd, qd, sd, zd = bf16_dev(x), u8_dev(qw), f16_dev(s), None if sym else f16_dev(z)
    y_eager = B.gq_w4a16_gemv(xd, qd, sd, zd, G, sym)
    torch.cuda.synchronize()
    ref = O.w4a16_reference(x, qw, s, None if sym else z, G, sym)
    wh = O.dequantize_packed(qw, s, None if sym else z, G, sym)
    assert_parity(bits16(y_eager), ref, O.bf16_to_f64(x), wh, f"[{N},{K}] M={M} G={G} eager")
    y_g = torch.empty_like(y_eager)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        B.gq_w4a16_gemv(xd, qd, sd, zd, G, sym, y=y_g)
        with torch.cuda.graph(g, stream=stream):
            B.gq_w4a16_gemv(xd, qd, sd, zd, G, sym, y=y_g)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for rep in range(3):
        y_g.zero_()
        g.replay()
        other = B.gq_w4a16_gemv(xd[:1], qd, sd, zd, G, sym)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_eager), f"replay {rep}"
        assert other.shape == (1, N)


@pytest.mark.parametrize("M", [5, 8, 16])
@pytest.mark.parametrize("N", [1, 15, 17])
def test_mfma_stream_tiny_row_counts(M, N):
    # one output row, one row short of a 16-row block, one row past it
    K, G = 4096, 64
    w, x = synth.small(N, K, M, seed=N * 31 + M)
    qw, s, z = _oracle_weights(w, G, False)
    _run(x, qw, s, z, G, False, f"[{N},{K}] M={M} asym G={G} (matrix cores, streaming)")


@pytest.mark.parametrize("M", [4, 5, 7, 12, 16])
@pytest.mark.parametrize("K", [512, 1024, 2048])
@pytest.mark.parametrize("sym,G", [(True, 32), (False, 64), (False, 128), (True, 256), (False, 512)])
def test_xreg_k_extents(M, K, sym, G):
    # x held in registers: one 512-wide column range per wave, K / 512 waves
    # per workgroup (1, 2, 4), a partial last row block (77 rows)
    assert B.gq_w4a16_gemv_workspace_size(M, K, 77, G, sym) == 0
    w, x = synth.small(77, K, M, seed=M * 101 + K + G)
    qw, s, z = _oracle_weights(w, G, sym)
    _run(x, qw, s, z, G, sym, f"[77,{K}] M={M} sym={sym} G={G} (x in registers)")


@pytest.mark.parametrize("M,N,K", [(9, 100003, 512), (6, 70001, 1024), (16, 36001, 2048)])
def test_xreg_many_row_blocks(M, N, K):
    # more row blocks than the grid has workgroups: every workgroup runs
    # several items, including the two-item tail, and alternates its tile
    # buffers; checked on the first, middle and last rows
    w, x = synth.small(N, K, M, seed=N + M)
    qw, s, z = _oracle_weights(w, 128, False)
    rows = np.r_[0:64, N // 2:N // 2 + 64, N - 67:N]
    _run(x, qw, s, z, 128, False, f"[{N},{K}] M={M} asym G=128 (x in registers, many rows)", rows=rows)


@pytest.mark.parametrize("M", [5, 8, 11, 16])
@pytest.mark.parametrize("K,sym,G", [(4352, True, 32), (4352, False, 64), (4608, False, 128),
                                     (5120, True, 256), (6144, False, 512), (14336, True, 1024)])
def test_xs_k_extents(M, K, sym, G):
    # long K with x streamed per item: items per row block not a multiple of
    # the 8 waves (17, 18, 20 of 256 columns: the last items of some waves lie
    # past K), every group class, a partial last row block (203 rows)
    assert B.gq_w4a16_gemv_workspace_size(M, K, 203, G, sym) == 0
    w, x = synth.small(203, K, M, seed=M * 7 + K + G)
    qw, s, z = _oracle_weights(w, G, sym)
    _run(x, qw, s, z, G, sym, f"[203,{K}] M={M} sym={sym} G={G} (x streamed)")


@pytest.mark.parametrize("M,N,K,sym,G", [(7, 300001, 512, False, 128), (13, 40003, 4352, True, 32)])
def test_many_row_block_groups(M, N, K, sym, G):
    # more than eight row blocks per workgroup, so the tile slots of a second
    # group of row blocks are used (register-resident x at K = 512, streamed x
    # at 4352); random packed weights and fp16 scales (and zero points),
    # checked on rows of the first and the last groups
    rng = np.random.default_rng(N + K)
    qw = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s = rng.uniform(1e-3, 1e-2, size=(N, K // G)).astype(np.float16).view(np.uint16)
    z = None if sym else rng.uniform(0, 15, size=(N, K // G)).astype(np.float16).view(np.uint16)
    x, _ = synth.activations(M, K, seed=N)
    rows = np.r_[0:64, 16 * 8 * 256:16 * 8 * 256 + 64, N - 67:N]
    _run(x, qw, s, z, G, sym, f"[{N},{K}] M={M} sym={sym} G={G} (two row-block groups)", rows=rows)


@pytest.mark.parametrize("M,N,K,sym,G", [(5, 6139, 4096, True, 32), (8, 6139, 4096, False, 128),
                                         (16, 6139, 4096, True, 32), (8, 12285, 4096, True, 32),
                                         (16, 12285, 4096, False, 64), (8, 6139, 4352, True, 32),
                                         (8, 12285, 4352, False, 128), (12, 6139, 4352, True, 32)])
def test_prefetch_paths_by_row_blocks_per_workgroup(M, N, K, sym, G):
    # 384 row blocks at K = 4096 on 256 workgroups (register-x kernel): half
    # of them take two (every prefetch issued), half one (the second prefetch
    # skipped); 768: three each, the loop's prefetches running past the last
    # row block; the last row block ragged.  At K = 4352 the streamed-x
    # kernel with one to three row blocks per workgroup, 8 rows (every
    # prefetch issued, also past the last item) and 16 rows (guarded).  Rows
    # at the start, around the second row block of the first workgroups, in
    # the middle and at the end.
    w, x = synth.small(N, K, M, seed=N + K + M)
    qw, s, z = _oracle_weights(w, G, sym)
    rows = np.r_[0:48, 4096 - 16:4096 + 48, N // 2:N // 2 + 32, N - 43:N]
    _run(x, qw, s, z, G, sym, f"[{N},{K}] M={M} sym={sym} G={G} (prefetch paths)", rows=rows)


@pytest.mark.parametrize("M", [5, 8, 16])
@pytest.mark.parametrize("N,K,sym,G", [(203, 1536, True, 32), (203, 3072, False, 128),
                                       (77, 2560, False, 512), (9001, 3072, True, 32)])
def test_lds_staged_k_between_register_sizes(M, N, K, sym, G):
    # K at most 4096 that is a multiple of 512 but not a power-of-two multiple:
    # the matrix-core kernel with x staged in LDS per workgroup (at M = 16 and
    # 9001 rows, two teams of 8 waves share one stage)
    assert B.gq_w4a16_gemv_workspace_size(M, K, N, G, sym) == 0
    w, x = synth.small(N, K, M, seed=N + K + M + G)
    qw, s, z = _oracle_weights(w, G, sym)
    rows = None if N < 1000 else np.r_[0:64, N // 2:N // 2 + 64, N - 67:N]
    _run(x, qw, s, z, G, sym, f"[{N},{K}] M={M} sym={sym} G={G} (x staged in LDS)", rows=rows)
