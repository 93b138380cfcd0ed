"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/gq.h, and rejects invalid arguments on the host before any
device call (the validation paths return without touching HIP)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT, read_golden
from oracle import gq_oracle as O
from w4a16_dequant_gemm_group_amd import binding as B

HEADER = os.path.join(ROOT, "include", "gq.h")
BENCH_HEADER = os.path.join(ROOT, "include", "gq_bench.h")


def header_functions(path=HEADER):
    src = open(path).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gq_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return B.lib()


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert len(names) == 20
    assert set(names) == set(B.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    bench = header_functions(BENCH_HEADER)
    assert set(bench) == set(B.BENCH_EXPORTS) and len(bench) == 4
    for n in bench:
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    for s in range(5):
        assert lib.gq_status_str(s).decode().startswith("GQ_")
    assert lib.gq_version() == 100


def test_packed_sizes_page_byte_counts():
    g = read_golden("p1_byte_counts.txt")
    for n, G, payload, meta, total in (map(int, r) for r in g["_rows"]):
        q, s, z = B.gq_packed_sizes(1, n, 4, G, False)
        assert (q, s + z, q + s + z) == (payload, meta, total)
    for N, K, G, sym in ((6144, 4096, 128, False), (4096, 14336, 32, True), (7, 96, 32, False)):
        assert B.gq_packed_sizes(N, K, 4, G, sym) == O.packed_sizes(N, K, G, sym)


FAKE = ctypes.c_void_p(4096)        # never dereferenced: every case below fails validation
FAKE_MIS = ctypes.c_void_p(4096 + 4)


def q(bits=4, g=128, sym=0):
    return B.GqQParams(bits, g, sym)


@pytest.mark.parametrize("args,expect", [
    # K not a multiple of the group size
    (dict(K=1000, p=q()), B.GQ_ERR_INVALID_ARG),
    # group size not a multiple of 32
    (dict(K=960, p=q(g=48)), B.GQ_ERR_INVALID_ARG),
    # M above the GEMV range
    (dict(M=17), B.GQ_ERR_INVALID_ARG),
    # negative sizes
    (dict(N=-1), B.GQ_ERR_INVALID_ARG),
    # asymmetric without zeros
    (dict(zeros=None), B.GQ_ERR_INVALID_ARG),
    # symmetric with zeros
    (dict(p=q(sym=1)), B.GQ_ERR_INVALID_ARG),
    # bits other than 4 on a packed path
    (dict(p=q(bits=8)), B.GQ_ERR_UNSUPPORTED),
    (dict(p=q(bits=9)), B.GQ_ERR_INVALID_ARG),
    # misaligned activation / output
    (dict(x=FAKE_MIS), B.GQ_ERR_MISALIGNED),
    (dict(y=FAKE_MIS), B.GQ_ERR_MISALIGNED),
    # NULL buffers
    (dict(qweight=None), B.GQ_ERR_INVALID_ARG),
])
def test_gemv_validation(lib, args, expect):
    a = dict(x=FAKE, M=1, K=4096, qweight=FAKE, scales=FAKE, zeros=FAKE, N=4096, p=q(), y=FAKE)
    a.update(args)
    st = lib.gq_w4a16_gemv(a["x"], a["M"], a["K"], a["qweight"], a["scales"], a["zeros"], a["N"],
                           a["p"], a["y"], None)
    assert st == expect
    if "M" not in args:
        st = lib.gq_w4a16_gemm(a["x"], a["M"], a["K"], a["qweight"], a["scales"], a["zeros"],
                               a["N"], a["p"], a["y"], None)
        assert st == expect


def test_empty_problems_are_noops(lib):
    # nothing to compute: returns OK without touching pointers or the device
    assert lib.gq_w4a16_gemv(None, 0, 4096, None, None, None, 4096, q(), None, None) == B.GQ_OK
    assert lib.gq_w4a16_gemm(None, 5, 4096, None, None, None, 0, q(), None, None) == B.GQ_OK
    assert lib.gq_quantize_groups(None, B.GQ_BF16, 0, 256, q(), None, None, None, None) == B.GQ_OK
    assert lib.gq_q4k_gemv(None, 0, 256, None, 8, None, None) == B.GQ_OK


def test_other_entry_point_validation(lib):
    L = lib
    assert L.gq_quantize_groups(FAKE, B.GQ_BF16, 4, 256, q(bits=1), FAKE, FAKE, FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_quantize_groups(FAKE, 7, 4, 256, q(), FAKE, FAKE, FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_quantize_groups(FAKE, B.GQ_BF16, 4, 256, q(sym=1), FAKE, FAKE, FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_pack_int4(FAKE, 4, 255, 0, FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_dequantize(FAKE, FAKE, FAKE, 4, 256, q(bits=3), FAKE, B.GQ_F32, None) == B.GQ_ERR_UNSUPPORTED
    assert L.gq_dequantize(FAKE, FAKE, FAKE, 4, 256, q(), FAKE, 9, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_q4k_quantize(FAKE, B.GQ_BF16, 4, 300, FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_q4k_gemv(FAKE, 1, 512, FAKE_MIS, 4, FAKE, None) == B.GQ_ERR_MISALIGNED
    assert L.gq_q4k_gemv(FAKE, 17, 512, FAKE, 4, FAKE, None) == B.GQ_ERR_INVALID_ARG


def test_gemv_workspace_size_and_validation(lib):
    # the split-K matrix-core path (4 <= M <= 16, G in {32, 64, 128k}, K % 256
    # == 0, where no scratch-free kernel takes the call: M = 4 beyond the
    # dot-product kernel's K, or K <= 4096 not a multiple of 512 for M > 4)
    # keeps ceil(K / 1024) * M * N fp32 partial sums; other calls need none
    assert B.gq_w4a16_gemv_workspace_size(16, 2304, 4096, 32, True) == 3 * 16 * 4096 * 4
    assert B.gq_w4a16_gemv_workspace_size(8, 3328, 203, 128) == 4 * 8 * 203 * 4
    assert B.gq_w4a16_gemv_workspace_size(4, 18176, 4096, 128) == 18 * 4 * 4096 * 4
    assert B.gq_w4a16_gemv_workspace_size(4, 16384, 4096, 128) == 0
    assert B.gq_w4a16_gemv_workspace_size(4, 4096, 4096, 128) == 0
    assert B.gq_w4a16_gemv_workspace_size(8, 4096, 4096, 128) == 0    # x in registers
    assert B.gq_w4a16_gemv_workspace_size(16, 4096, 4096, 32, True) == 0
    assert B.gq_w4a16_gemv_workspace_size(8, 14336, 4096, 32, True) == 0   # x streamed per item
    assert B.gq_w4a16_gemv_workspace_size(16, 14336, 4096, 32, True) == 0
    assert B.gq_w4a16_gemv_workspace_size(16, 14080, 4096, 32, True) == 0
    assert B.gq_w4a16_gemv_workspace_size(8, 4352, 4096, 128) == 0
    assert B.gq_w4a16_gemv_workspace_size(8, 3072, 4096, 128) == 0    # x staged in LDS
    assert B.gq_w4a16_gemv_workspace_size(3, 4096, 4096, 128) == 0
    assert B.gq_w4a16_gemv_workspace_size(1, 4096, 4096, 128) == 0
    assert B.gq_w4a16_gemv_workspace_size(8, 6528, 203, 128) == 0   # K % 256 != 0
    assert B.gq_w4a16_gemv_workspace_size(8, 6528, 203, 96) == 0    # G outside 32, 64, 128k
    assert B.gq_w4a16_gemv_workspace_size(0, 4352, 4096, 128) == 0
    nbytes = ctypes.c_size_t()
    assert lib.gq_w4a16_gemv_workspace_size(17, 4096, 64, q(), ctypes.byref(nbytes)) == B.GQ_ERR_INVALID_ARG
    assert lib.gq_w4a16_gemv_workspace_size(8, 4096, 64, q(g=48), ctypes.byref(nbytes)) == B.GQ_ERR_INVALID_ARG
    assert lib.gq_w4a16_gemv_workspace_size(8, 4096, 64, q(), None) == B.GQ_ERR_INVALID_ARG
    # a needed workspace that is missing, too small or misaligned is rejected before any device call
    need = B.gq_w4a16_gemv_workspace_size(8, 3328, 4096, 128)
    assert need > 0
    args = (FAKE, 8, 3328, FAKE, FAKE, FAKE, 4096, q(), FAKE)
    assert lib.gq_w4a16_gemv_ws(*args, None, need, None) == B.GQ_ERR_INVALID_ARG
    assert lib.gq_w4a16_gemv_ws(*args, FAKE, need - 4, None) == B.GQ_ERR_INVALID_ARG
    assert lib.gq_w4a16_gemv_ws(*args, FAKE_MIS, need, None) == B.GQ_ERR_MISALIGNED
    # the plain GEMV checks still apply
    assert lib.gq_w4a16_gemv_ws(FAKE, 17, 3328, FAKE, FAKE, FAKE, 4096, q(), FAKE, FAKE, need, None) == B.GQ_ERR_INVALID_ARG


def test_bench_entry_point_validation(lib):
    L = lib
    # bf16 GEMV: M in 0..4, K a multiple of 8, byte limits, alignment
    assert L.gq_bf16_gemv(FAKE, 5, 4096, FAKE, 64, FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_bf16_gemv(FAKE, 1, 4092, FAKE, 64, FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_bf16_gemv(FAKE, 1, 4096, FAKE, -1, FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_bf16_gemv(FAKE, 1, 4096, FAKE, 1 << 18, FAKE, None) == B.GQ_ERR_UNSUPPORTED
    # x staged in LDS: M * round_up(K, 2048) activations must fit 32768
    assert L.gq_bf16_gemv(FAKE, 3, 14336, FAKE, 64, FAKE, None) == B.GQ_ERR_UNSUPPORTED
    assert L.gq_bf16_gemv(FAKE, 1, 32776, FAKE, 64, FAKE, None) == B.GQ_ERR_UNSUPPORTED
    assert L.gq_bf16_gemv(FAKE_MIS, 1, 4096, FAKE, 64, FAKE, None) == B.GQ_ERR_MISALIGNED
    assert L.gq_bf16_gemv(FAKE, 1, 4096, FAKE_MIS, 64, FAKE, None) == B.GQ_ERR_MISALIGNED
    assert L.gq_bf16_gemv(FAKE, 1, 4096, FAKE, 64, ctypes.c_void_p(4097), None) == B.GQ_ERR_MISALIGNED
    assert L.gq_bf16_gemv(None, 1, 4096, FAKE, 64, FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_bf16_gemv(None, 0, 4096, None, 64, None, None) == B.GQ_OK
    # stream read: whole 16-byte words, bounded size, alignment
    assert L.gq_stream_read(FAKE, 24, FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_stream_read(FAKE, -16, FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_stream_read(FAKE, (1 << 38) + 16, FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_stream_read(FAKE_MIS, 64, FAKE, None) == B.GQ_ERR_MISALIGNED
    assert L.gq_stream_read(FAKE, 64, ctypes.c_void_p(4098), None) == B.GQ_ERR_MISALIGNED
    assert L.gq_stream_read(FAKE, 64, None, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_stream_read(None, 0, None, None) == B.GQ_OK
    # issue-rate probes: fixed vector-work counts, bounded iterations and grid, alignment
    assert L.gq_probe_mfma_valu(16, 10, 1, FAKE, FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_probe_mfma_valu(32, 0, 1, FAKE, FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_probe_mfma_valu(32, 10, 0, FAKE, FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_probe_mfma_valu(32, 10, 1, None, FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_probe_mfma_valu(32, 10, 1, ctypes.c_void_p(4100), FAKE, None) == B.GQ_ERR_MISALIGNED
    assert L.gq_probe_lds_read(17, 10, 1, FAKE, FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_probe_lds_read(8, (1 << 20) + 1, 1, FAKE, FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_probe_lds_read(8, 10, 1, FAKE, ctypes.c_void_p(4098), None) == B.GQ_ERR_MISALIGNED



def test_ingest_validation(lib):
    L = lib
    assert L.gq_ingest_group_major(FAKE, FAKE, 4, 48, 64, FAKE, FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_ingest_group_major(FAKE, FAKE, 0, 32, 64, FAKE, FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_ingest_group_major(FAKE, FAKE, 4, 32, -1, FAKE, FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_ingest_group_major(None, FAKE, 4, 32, 64, FAKE, FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_ingest_group_major(FAKE, FAKE, 4, 32, 64, FAKE_MIS, FAKE, None) == B.GQ_ERR_MISALIGNED
    assert L.gq_ingest_group_major(None, None, 4, 32, 0, None, None, None) == B.GQ_OK



def test_f16_entry_point_validation(lib):
    L = lib
    # the fp16 entry points validate like the bf16 ones (every shape is supported)
    assert L.gq_w4a16_gemv_f16(FAKE, 17, 4096, FAKE, FAKE, FAKE, 4096, q(), FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_w4a16_gemv_f16(FAKE_MIS, 1, 4096, FAKE, FAKE, FAKE, 64, q(), FAKE, None) == B.GQ_ERR_MISALIGNED
    assert L.gq_w4a16_gemm_f16(FAKE_MIS, 64, 4096, FAKE, FAKE, FAKE, 4096, q(), FAKE, None) == B.GQ_ERR_MISALIGNED
    assert L.gq_w4a16_gemm_f16(FAKE, 64, 4096, FAKE, FAKE, None, 4096, q(), FAKE, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_w4a16_gemm_f16(FAKE, 64, 4096, FAKE, FAKE, FAKE, 4096, q(bits=8), FAKE, None) == B.GQ_ERR_UNSUPPORTED
    need = B.gq_w4a16_gemv_workspace_size(16, 2304, 4096, 128)
    assert need > 0
    args = (FAKE, 16, 2304, FAKE, FAKE, FAKE, 4096, q(), FAKE)
    assert L.gq_w4a16_gemv_f16_ws(*args, None, need, None) == B.GQ_ERR_INVALID_ARG
    assert L.gq_w4a16_gemv_f16_ws(*args, FAKE_MIS, need, None) == B.GQ_ERR_MISALIGNED


def test_gemm_workspace_size_and_validation(lib):
    """The split covers the last round of 256 x 256 tiles when it fills at most
    half of the compute units (256 when no device is present): 16 bytes of
    handshake words per split tile (padded to 256) plus a 256 x 256 fp32 tile."""
    def ws(M, K, N, G=128, sym=False):
        return B.gq_w4a16_gemm_workspace_size(M, K, N, G, sym)
    tile = 256 * 256 * 4

    def split(t):  # handshake words padded to 256 bytes, then the partial tiles
        return -(-16 * t // 256) * 256 + t * tile
    assert ws(2048, 4096, 4096) == split(128) == 2048 + 128 * tile   # o: 128 tiles, all split
    assert ws(2048, 14336, 4096) == split(128)                      # down
    assert ws(2048, 4096, 6144) == 0                                # qkv: 192 tiles > 128
    assert ws(2048, 4096, 28672) == split(128)                      # gate_up: 896 = 3 x 256 + 128
    assert ws(512, 2048, 512) == split(4) == 256 + 4 * tile
    assert ws(256, 256, 256) == 0                            # halves too short to split
    assert ws(2048, 4096, 4096, 32) == 0                     # group 32: the generic kernel
    assert ws(300, 4128, 200, 96, True) == 0                 # K % 64 == 32
    assert ws(0, 4096, 4096) == 0
    nbytes = ctypes.c_size_t()
    assert lib.gq_w4a16_gemm_workspace_size(64, 4096, 64, q(g=48), ctypes.byref(nbytes)) == B.GQ_ERR_INVALID_ARG
    assert lib.gq_w4a16_gemm_workspace_size(64, 4096, 64, q(), None) == B.GQ_ERR_INVALID_ARG
    assert lib.gq_w4a16_gemm_workspace_size(64, 1 << 23, 64, q(), ctypes.byref(nbytes)) == B.GQ_ERR_UNSUPPORTED
    need = ws(2048, 4096, 4096)
    args = (FAKE, 2048, 4096, FAKE, FAKE, FAKE, 4096, q(), FAKE)
    for fn in (lib.gq_w4a16_gemm_ws, lib.gq_w4a16_gemm_f16_ws):
        assert fn(*args, None, need, None) == B.GQ_ERR_INVALID_ARG
        assert fn(*args, FAKE, need - 16, None) == B.GQ_ERR_INVALID_ARG
        assert fn(*args, FAKE_MIS, need, None) == B.GQ_ERR_MISALIGNED


def test_binding_checks_tensors_before_any_call():
    """The binding rejects wrong shapes, dtypes and devices of inputs and of
    caller-supplied outputs before it calls the library (CPU tensors here: the
    shape and dtype checks come first, the device check last)."""
    import torch
    N, K, G = 64, 512, 128
    x = torch.zeros((2, K), dtype=torch.bfloat16)
    qw = torch.zeros((N, K // 2), dtype=torch.uint8)
    sc = torch.zeros((N, K // G), dtype=torch.float16)
    zr = torch.zeros((N, K // G), dtype=torch.float16)
    cases = [
        (dict(y=torch.zeros((2, N - 1), dtype=torch.bfloat16)), ValueError, "y has shape"),
        (dict(y=torch.zeros((2, N), dtype=torch.float16)), TypeError, "y: dtype"),
        (dict(scales=torch.zeros((N, K // G - 1), dtype=torch.float16)), ValueError, "scales has shape"),
        (dict(zeros=torch.zeros((N + 1, K // G), dtype=torch.float16)), ValueError, "zeros has shape"),
        (dict(zeros=None), ValueError, "need zeros"),
        (dict(qweight=torch.zeros((N, K // 4), dtype=torch.uint8)), ValueError, "does not match K"),
        (dict(x=torch.zeros((17, K), dtype=torch.bfloat16)), ValueError, "M <= 16"),
        (dict(group_size=96), ValueError, "group_size"),
        (dict(workspace=torch.zeros(16, dtype=torch.int32)), TypeError, "workspace: dtype"),
        (dict(), ValueError, "must be a GPU tensor"),
    ]
    for over, exc, msg in cases:
        a = dict(x=x, qweight=qw, scales=sc, zeros=zr, group_size=G, y=None, workspace=None)
        a.update(over)
        with pytest.raises(exc, match=msg):
            B.gq_w4a16_gemv(a["x"], a["qweight"], a["scales"], a["zeros"], a["group_size"], False,
                            y=a["y"], workspace=a["workspace"])
    with pytest.raises(ValueError, match="y has shape"):
        B.gq_w4a16_gemm(x, qw, sc, zr, G, False, y=torch.zeros((3, N), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="blocks has shape"):
        B.gq_q4k_gemv(x, torch.zeros((N, 1, 144), dtype=torch.uint8))
    with pytest.raises(ValueError, match="y has shape"):
        B.gq_q4k_gemv(x, torch.zeros((N, 2, 144), dtype=torch.uint8), y=torch.zeros((2, 7), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out has shape"):
        B.gq_dequantize(qw, sc, zr, G, False, out=torch.zeros((N, K - 2), dtype=torch.float32))
    with pytest.raises(ValueError, match="codes has shape"):
        B.gq_quantize_groups(torch.zeros((N, K), dtype=torch.bfloat16), 4, G, False,
                             codes=torch.zeros((N, K - 1), dtype=torch.uint8))
    with pytest.raises(ValueError, match="qweight has shape"):
        B.gq_pack_int4(torch.zeros((N, K), dtype=torch.uint8), qweight=torch.zeros((N, K), dtype=torch.uint8))
    with pytest.raises(ValueError, match="blocks has shape"):
        B.gq_q4k_quantize(torch.zeros((N, K), dtype=torch.float32), blocks=torch.zeros((N, 3, 144), dtype=torch.uint8))
