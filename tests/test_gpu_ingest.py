"""GPU checks of gq_ingest_group_major: the "量化" chapter's group-major layout
(codes int8 [n_groups, group, N], scales fp16 [n_groups, N]) converted to the
canonical [N, K/2] + [N, K/G] form must equal the oracle's conversion byte for
byte, and the fused GEMV / GEMM on the converted weight must reproduce the
chapter's group-by-group product."""
import numpy as np
import pytest
import torch

from gpu_util import announce, assert_parity, bf16_dev, bits16, device
from oracle import gq_oracle as O
from w4a16_dequant_gemm_group_amd import binding as B
import synth

pytestmark = pytest.mark.gpu


def _page_case(ng, g, n, seed):
    """Symmetric 4-bit codes and fp16 scales in the chapter's layout, from a
    synthetic weight quantized by the oracle (so codes span -8..7)."""
    w, _ = synth.weights(n, ng * g, seed=seed)
    codes, s, _ = O.quantize_to_storage(w, 4, g, True)          # [N, K], [N, ng]
    codes_gkn = np.ascontiguousarray(codes.T.reshape(ng, g, n).astype(np.int8))
    scales_gn = np.ascontiguousarray(s.T)
    return codes_gkn, scales_gn


@pytest.mark.parametrize("ng,g,n", [(4, 32, 64), (7, 64, 200), (3, 128, 1), (32, 128, 4096), (9, 32, 130)])
def test_ingest_matches_oracle_bytes(ng, g, n):
    announce(f"ingest ng={ng} g={g} N={n}")
    codes, scales = _page_case(ng, g, n, seed=ng * g + n)
    c_dev = torch.from_numpy(codes).to(device())
    s_dev = torch.from_numpy(scales.view(np.int16)).view(torch.float16).to(device())
    qw, so = B.gq_ingest_group_major(c_dev, s_dev)
    torch.cuda.synchronize()
    q_ref, s_ref = O.ingest_group_major(codes, scales)
    assert np.array_equal(qw.cpu().numpy(), q_ref)
    assert np.array_equal(bits16(so), s_ref)


@pytest.mark.parametrize("m", [1, 8, 96])
def test_matmuls_on_ingested_weights(m):
    announce(f"ingested weights through the matmuls M={m}")
    ng, g, n = 16, 128, 320
    codes, scales = _page_case(ng, g, n, seed=77)
    c_dev = torch.from_numpy(codes).to(device())
    s_dev = torch.from_numpy(scales.view(np.int16)).view(torch.float16).to(device())
    qw, so = B.gq_ingest_group_major(c_dev, s_dev)
    x, _ = synth.activations(m, ng * g, seed=5 + m, n_outlier_channels=2)
    fn = B.gq_w4a16_gemv if m <= 16 else B.gq_w4a16_gemm
    y = fn(bf16_dev(x), qw, so, None, g, True)
    torch.cuda.synchronize()
    xf = O.bf16_to_f64(x)
    s = O.f16_to_f64(scales)
    page = np.zeros((m, n))
    for gi in range(ng):   # the chapter's fused form on its own layout
        page += xf[:, gi * g:(gi + 1) * g] @ (codes[gi].astype(np.float64) * s[gi])
    q_ref, s_ref = O.ingest_group_major(codes, scales)
    wh = O.dequantize_packed(q_ref, s_ref, None, g, True)
    assert_parity(bits16(y), page, xf, wh, f"ingested [{n},{ng * g}] M={m}")
