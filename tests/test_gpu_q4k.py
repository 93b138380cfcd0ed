"""GPU parity of the super-block format: quantize bit-exact (all 144 bytes of
every block), fused GEMV within the parity bar."""
import numpy as np
import pytest
import torch

from gpu_util import announce, assert_parity, bf16_dev, bits16, device, u8_dev
from oracle import gq_oracle as O
from w4a16_dequant_gemm_group_amd import binding as B
import synth

pytestmark = pytest.mark.gpu


def test_quantize_bit_exact_with_edge_blocks():
    w, _ = synth.weights(40, 1024, seed=21)
    wf = O.bf16_to_f64(w)
    wf[0, :256] = 0.0                       # all-zero block
    wf[1, 32:64] = 0.0                      # all-zero sub-block
    wf[2, :256] = np.abs(wf[2, :256])       # no negative values: dmin = 0
    wf[3, :256] *= 1e-3                     # tiny block: d near fp16 subnormals
    wb = synth.f32_to_bf16_bits(wf.astype(np.float32))
    announce("q4k quantize [40,1024] edge blocks")
    blocks = B.gq_q4k_quantize(bf16_dev(wb))
    torch.cuda.synchronize()
    ref = O.q4k_encode(O.q4k_quantize(O.bf16_to_f64(wb)))
    got = blocks.cpu().numpy()
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"blocks differ at {bad[:5]}"


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
def test_quantize_other_dtypes(dtype):
    rng = np.random.default_rng(3)
    w = rng.normal(0, 0.1, size=(9, 512)).astype(np.float32)
    wd = torch.from_numpy(w).to(device()).to(dtype)
    blocks = B.gq_q4k_quantize(wd)
    ref = O.q4k_encode(O.q4k_quantize(wd.float().cpu().numpy().astype(np.float64)))
    assert np.array_equal(blocks.cpu().numpy(), ref)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 16])
@pytest.mark.parametrize("N,K", [(77, 2304), (64, 256), (33, 18432), (1031, 4096), (1031, 10496),
                                 (37, 28672), (129, 73728)])
def test_gemv_small(M, N, K):
    """M = 1..4 take the streaming kernel while every activation row fits one
    compute unit's LDS (4352 bytes per row and 2048-step): a ragged last step at
    2304 and 256, several row pairs per wave at 1031 rows, one workgroup per
    compute unit from four steps on, x staged in more than one pass at M = 1
    with 28672 and 73728 (36 steps) and at M = 2..4 with 18432 and beyond; M = 2
    at 73728 and M = 3, 4 from 28672 on take the per-workgroup kernel.  M = 16
    takes the matrix-core kernel where K is a multiple of 512 (x in chunks of
    4096 columns beyond 4096) and the per-workgroup kernel at 2304, 256 and
    10496."""
    w, x = synth.small(N, K, M, seed=N + M)
    blocks = O.q4k_encode(O.q4k_quantize(O.bf16_to_f64(w)))
    y = B.gq_q4k_gemv(bf16_dev(x), u8_dev(blocks))
    torch.cuda.synchronize()
    ref = O.q4k_reference(x, blocks)
    wh = O.q4k_dequantize_fields(O.q4k_decode(blocks))
    assert_parity(bits16(y), ref, O.bf16_to_f64(x), wh, f"q4k gemv [{N},{K}] M={M}")


@pytest.mark.parametrize("M", [5, 8, 9, 13, 16])
@pytest.mark.parametrize("N,K", [(77, 4096), (1031, 4096), (33, 14336), (16, 2048), (203, 8192),
                                 (3, 512), (21, 2560)])
def test_gemv_matrix_cores(M, N, K):
    """M = 5..16 on the matrix cores (one MFMA per sub-block and 16 rows): a
    partial last row block (77, 33, 21, 3 rows), several row blocks per
    workgroup (1031), x in chunks (14336: two chunks of 8192 with 8 staged
    rows, four of 4096 with 16, the last partial), items past K (2048, 2560,
    512), 8192 with 8 staged rows in one stage and with 16 in two."""
    w, x = synth.small(N, K, M, seed=N + K + M)
    blocks = O.q4k_encode(O.q4k_quantize(O.bf16_to_f64(w)))
    y = B.gq_q4k_gemv(bf16_dev(x), u8_dev(blocks))
    torch.cuda.synchronize()
    ref = O.q4k_reference(x, blocks)
    wh = O.q4k_dequantize_fields(O.q4k_decode(blocks))
    assert_parity(bits16(y), ref, O.bf16_to_f64(x), wh, f"q4k gemv [{N},{K}] M={M} (matrix cores)")


@pytest.mark.parametrize("name", ["down", "gate_up"])
@pytest.mark.parametrize("M", [1, 4, 8, 16])
def test_full_size(name, M):
    """Full-size super-block quantize + GEMV at M = 1 and 4 (the streaming
    kernel) and 8 and 16 (the matrix cores; down in chunks of x): every
    block's 144 bytes and every output row against the oracle, in row
    chunks."""
    w, x = synth.q4k_case(name, M)
    announce(f"q4k {name} {w.shape} M={M}, all rows")
    blocks = B.gq_q4k_quantize(bf16_dev(w))
    y = B.gq_q4k_gemv(bf16_dev(x), blocks)
    torch.cuda.synchronize()
    got = blocks.cpu().numpy()
    N = w.shape[0]
    ref = np.empty((M, N))
    wmax = 0.0
    for r0 in range(0, N, 2048):
        r1 = min(N, r0 + 2048)
        ref_blocks = O.q4k_encode(O.q4k_quantize(O.bf16_to_f64(w[r0:r1])))
        assert np.array_equal(got[r0:r1], ref_blocks), r0
        wh = O.q4k_dequantize_fields(O.q4k_decode(ref_blocks))
        wmax = max(wmax, float(np.abs(wh).max()))
        ref[:, r0:r1] = O.matmul_groupwise(O.bf16_to_f64(x), wh, O.Q4K_SUB)
    assert_parity(bits16(y), ref, O.bf16_to_f64(x), np.array([[wmax]]),
                  f"q4k {name} {w.shape} M={M} full, all rows")


@pytest.mark.parametrize("M,N,K", [(7, 300001, 512), (13, 40003, 4352)])
def test_gemv_many_row_block_groups(M, N, K):
    """More than eight row blocks per workgroup on the matrix cores (x in
    registers at K = 512, streamed per block at K = 4352), so a second group of
    tile slots is used: blocks quantized on the GPU from seeded N(0, 0.02)
    weights, checked bit-exact and through the GEMV on rows of the first and
    last groups."""
    gen = torch.Generator(device=device()).manual_seed(N + K)
    wd = (torch.randn((N, K), generator=gen, device=device()) * 0.02).to(torch.bfloat16)
    x, _ = synth.activations(M, K, seed=N)
    announce(f"q4k gemv [{N},{K}] M={M}, two row-block groups")
    blocks = B.gq_q4k_quantize(wd)
    y = B.gq_q4k_gemv(bf16_dev(x), blocks)
    torch.cuda.synchronize()
    rows = np.r_[0:64, N - 67:N]
    wr = wd[torch.from_numpy(rows).to(device())].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    del wd
    ref_blocks = O.q4k_encode(O.q4k_quantize(O.bf16_to_f64(wr)))
    assert np.array_equal(blocks.cpu().numpy()[rows], ref_blocks)
    ref = O.q4k_reference(x, ref_blocks)
    wh = O.q4k_dequantize_fields(O.q4k_decode(ref_blocks))
    assert_parity(bits16(y)[:, rows], ref, O.bf16_to_f64(x), wh, f"q4k gemv [{N},{K}] M={M} (two groups), sampled")
