"""Thin ctypes binding of libgq (``include/gq.h``), same names as the C ABI.

The functions here only marshal arguments: they check dtypes, devices and
contiguity of torch tensors, allocate missing outputs with torch (device memory
plumbing), and pass raw pointers plus the current HIP stream to the library.
Every step of the computation runs in the library's kernels; there is no
fallback path.  A missing ``libgq.so`` raises immediately.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgq.so")

GQ_OK, GQ_ERR_INVALID_ARG, GQ_ERR_UNSUPPORTED, GQ_ERR_MISALIGNED, GQ_ERR_HIP = range(5)
GQ_F32, GQ_F16, GQ_BF16 = 0, 1, 2

# Every entry point declared in include/gq.h.
EXPORTS = (
    "gq_status_str", "gq_version", "gq_packed_sizes", "gq_quantize_groups", "gq_pack_int4",
    "gq_dequantize", "gq_w4a16_gemv", "gq_w4a16_gemv_workspace_size", "gq_w4a16_gemv_ws",
    "gq_w4a16_gemm", "gq_q4k_quantize", "gq_q4k_gemv", "gq_ingest_group_major",
    "gq_w4a16_gemv_f16", "gq_w4a16_gemm_f16",
)
# comparators and probes (include/gq_bench.h)
BENCH_EXPORTS = ("gq_bf16_gemv", "gq_stream_read")


class GqQParams(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("symmetric", ctypes.c_int32)]


class GqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib().gq_status_str(status).decode()}")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libgq.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m w4a16_dequant_gemm_group_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    p, i64, i32, c = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    Q = GqQParams
    L.gq_status_str.restype = ctypes.c_char_p
    L.gq_status_str.argtypes = [c]
    L.gq_version.restype = i32
    L.gq_version.argtypes = []
    sig = {
        "gq_packed_sizes": [i64, i64, Q, ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(i64)],
        "gq_quantize_groups": [p, c, i64, i64, Q, p, p, p, p],
        "gq_pack_int4": [p, i64, i64, i32, p, p],
        "gq_dequantize": [p, p, p, i64, i64, Q, p, c, p],
        "gq_w4a16_gemv": [p, i64, i64, p, p, p, i64, Q, p, p],
        "gq_w4a16_gemv_workspace_size": [i64, i64, i64, Q, ctypes.POINTER(ctypes.c_size_t)],
        "gq_w4a16_gemv_ws": [p, i64, i64, p, p, p, i64, Q, p, p, ctypes.c_size_t, p],
        "gq_w4a16_gemm": [p, i64, i64, p, p, p, i64, Q, p, p],
        "gq_q4k_quantize": [p, c, i64, i64, p, p],
        "gq_q4k_gemv": [p, i64, i64, p, i64, p, p],
        "gq_bf16_gemv": [p, i64, i64, p, i64, p, p],
        "gq_ingest_group_major": [p, p, i64, i64, i64, p, p, p],
        "gq_w4a16_gemv_f16": [p, i64, i64, p, p, p, i64, Q, p, p],
        "gq_w4a16_gemm_f16": [p, i64, i64, p, p, p, i64, Q, p, p],
        "gq_stream_read": [p, i64, p, p],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = c
    _lib = L
    return L


def _check(status: int, where: str) -> None:
    if status != GQ_OK:
        raise GqError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t: torch.Tensor, name: str, dtypes, dev=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")


_DT = {torch.float32: GQ_F32, torch.float16: GQ_F16, torch.bfloat16: GQ_BF16}


def qparams(bits: int = 4, group_size: int = 128, symmetric: bool = False) -> GqQParams:
    return GqQParams(int(bits), int(group_size), int(bool(symmetric)))


def gq_version() -> int:
    return int(lib().gq_version())


def gq_packed_sizes(N: int, K: int, bits: int = 4, group_size: int = 128, symmetric: bool = False):
    """(qweight_bytes, scale_bytes, zero_bytes) of an [N, K] weight."""
    q, s, z = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib().gq_packed_sizes(N, K, qparams(bits, group_size, symmetric),
                                 ctypes.byref(q), ctypes.byref(s), ctypes.byref(z)), "gq_packed_sizes")
    return q.value, s.value, z.value


def gq_quantize_groups(w: torch.Tensor, bits: int = 4, group_size: int = 128,
                       symmetric: bool = False, codes=None, scales=None, zeros=None, stream=None):
    """w [N, K] (bf16/fp16/fp32) -> (codes u8/i8 [N,K], scales fp16 [N,K/G], zeros fp16 or None)."""
    _need(w, "w", tuple(_DT))
    N, K = w.shape
    dev = w.device
    ng = K // group_size if group_size > 0 else 0
    if codes is None:
        codes = torch.empty((N, K), dtype=torch.int8 if symmetric else torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((N, ng), dtype=torch.float16, device=dev)
    if zeros is None and not symmetric:
        zeros = torch.empty((N, ng), dtype=torch.float16, device=dev)
    _check(lib().gq_quantize_groups(_ptr(w), _DT[w.dtype], N, K, qparams(bits, group_size, symmetric),
                                    _ptr(codes), _ptr(scales), _ptr(zeros), _stream(stream)),
           "gq_quantize_groups")
    return codes, scales, zeros


def gq_pack_int4(codes: torch.Tensor, symmetric: bool = False, qweight=None, stream=None):
    """codes [N, K] -> qweight uint8 [N, K/2] (low nibble = even k)."""
    _need(codes, "codes", (torch.uint8, torch.int8))
    N, K = codes.shape
    if qweight is None:
        qweight = torch.empty((N, K // 2), dtype=torch.uint8, device=codes.device)
    _check(lib().gq_pack_int4(_ptr(codes), N, K, int(bool(symmetric)), _ptr(qweight), _stream(stream)),
           "gq_pack_int4")
    return qweight


def gq_dequantize(qweight: torch.Tensor, scales: torch.Tensor, zeros: Optional[torch.Tensor],
                  group_size: int = 128, symmetric: bool = False, out_dtype=torch.float32,
                  out=None, stream=None):
    """Packed INT4 -> W^ [N, K] in out_dtype (fp32 exact; bf16/fp16 nearest-even)."""
    _need(qweight, "qweight", (torch.uint8,))
    _need(scales, "scales", (torch.float16,))
    N, K = qweight.shape[0], qweight.shape[1] * 2
    if out is None:
        out = torch.empty((N, K), dtype=out_dtype, device=qweight.device)
    _check(lib().gq_dequantize(_ptr(qweight), _ptr(scales), _ptr(zeros), N, K,
                               qparams(4, group_size, symmetric), _ptr(out), _DT[out.dtype],
                               _stream(stream)), "gq_dequantize")
    return out


def _matmul(fn, name, x, qweight, scales, zeros, group_size, symmetric, y, stream,
            xdtype=torch.bfloat16):
    _need(x, "x", (xdtype,))
    _need(qweight, "qweight", (torch.uint8,), x.device)
    _need(scales, "scales", (torch.float16,), x.device)
    if zeros is not None:
        _need(zeros, "zeros", (torch.float16,), x.device)
    M, K = x.shape
    N = qweight.shape[0]
    if qweight.shape[1] * 2 != K:
        raise ValueError(f"qweight {tuple(qweight.shape)} does not match K={K}")
    if y is None:
        y = torch.empty((M, N), dtype=xdtype, device=x.device)
    _check(fn(_ptr(x), M, K, _ptr(qweight), _ptr(scales), _ptr(zeros), N,
              qparams(4, group_size, symmetric), _ptr(y), _stream(stream)), name)
    return y


def gq_w4a16_gemv_workspace_size(M: int, K: int, N: int, group_size: int = 128,
                                 symmetric: bool = False) -> int:
    """Bytes of scratch gq_w4a16_gemv_ws needs (0: none)."""
    b = ctypes.c_size_t()
    _check(lib().gq_w4a16_gemv_workspace_size(M, K, N, qparams(4, group_size, symmetric),
                                              ctypes.byref(b)), "gq_w4a16_gemv_workspace_size")
    return int(b.value)


def _capturing(stream) -> bool:
    if stream is None:
        return torch.cuda.is_current_stream_capturing()
    if not hasattr(stream, "cuda_stream"):
        return True  # a raw handle: take the path that is safe under capture
    with torch.cuda.stream(stream):
        return torch.cuda.is_current_stream_capturing()


def gq_w4a16_gemv(x, qweight, scales, zeros, group_size: int = 128, symmetric: bool = False,
                  y=None, stream=None, workspace=None):
    """Fused W4A16 GEMV, x bf16 [M<=16, K] -> y bf16 [M, N].

    Eager calls use gq_w4a16_gemv (library scratch).  When the call needs
    scratch (gq_w4a16_gemv_workspace_size > 0) and the stream is being
    captured, or `workspace` (a uint8 GPU tensor) is given, the scratch comes
    from torch's allocator on the call's stream (or is `workspace`) and the call
    goes to gq_w4a16_gemv_ws: a captured graph then holds no pointer into
    library scratch that a later call could reallocate.  Both give the same
    bits."""
    _need(x, "x", (torch.bfloat16,))
    M, K = x.shape
    N = qweight.shape[0]
    need = gq_w4a16_gemv_workspace_size(M, K, N, group_size, symmetric) if M <= 16 else 0
    if workspace is None and (need == 0 or not _capturing(stream)):
        return _matmul(lib().gq_w4a16_gemv, "gq_w4a16_gemv", x, qweight, scales, zeros,
                       group_size, symmetric, y, stream)
    if workspace is None:
        # allocated on the call's stream, so the allocator hands this memory to
        # other work only after the call's kernels on that stream
        if stream is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        else:
            with torch.cuda.stream(stream):
                workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _need(workspace, "workspace", (torch.uint8,), x.device)
    ws, nbytes = workspace, workspace.numel()

    def fn(*a):
        return lib().gq_w4a16_gemv_ws(*a[:9], _ptr(ws), nbytes, a[9])
    return _matmul(fn, "gq_w4a16_gemv_ws", x, qweight, scales, zeros, group_size, symmetric,
                   y, stream)


def gq_w4a16_gemm(x, qweight, scales, zeros, group_size: int = 128, symmetric: bool = False,
                  y=None, stream=None):
    """Fused W4A16 GEMM (bf16 MFMA), x bf16 [M, K] -> y bf16 [M, N]."""
    return _matmul(lib().gq_w4a16_gemm, "gq_w4a16_gemm", x, qweight, scales, zeros,
                   group_size, symmetric, y, stream)


def gq_w4a16_gemv_f16(x, qweight, scales, zeros, group_size: int = 128, symmetric: bool = False,
                      y=None, stream=None):
    """Fused W4A16 GEMV with fp16 activations, x fp16 [M<=16, K] -> y fp16 [M, N]."""
    return _matmul(lib().gq_w4a16_gemv_f16, "gq_w4a16_gemv_f16", x, qweight, scales, zeros,
                   group_size, symmetric, y, stream, torch.float16)


def gq_w4a16_gemm_f16(x, qweight, scales, zeros, group_size: int = 128, symmetric: bool = False,
                      y=None, stream=None):
    """Fused W4A16 GEMM with fp16 activations (fp16 MFMA), x fp16 [M, K] -> y fp16 [M, N]."""
    return _matmul(lib().gq_w4a16_gemm_f16, "gq_w4a16_gemm_f16", x, qweight, scales, zeros,
                   group_size, symmetric, y, stream, torch.float16)


def gq_q4k_quantize(w: torch.Tensor, blocks=None, stream=None):
    """w [N, K] (K % 256 == 0) -> blocks uint8 [N, K/256, 144]."""
    _need(w, "w", tuple(_DT))
    N, K = w.shape
    if blocks is None:
        blocks = torch.empty((N, K // 256, 144), dtype=torch.uint8, device=w.device)
    _check(lib().gq_q4k_quantize(_ptr(w), _DT[w.dtype], N, K, _ptr(blocks), _stream(stream)),
           "gq_q4k_quantize")
    return blocks


def gq_q4k_gemv(x: torch.Tensor, blocks: torch.Tensor, y=None, stream=None):
    """Fused GEMV over super-block weights, x bf16 [M<=16, K] -> y bf16 [M, N]."""
    _need(x, "x", (torch.bfloat16,))
    _need(blocks, "blocks", (torch.uint8,), x.device)
    M, K = x.shape
    N = blocks.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check(lib().gq_q4k_gemv(_ptr(x), M, K, _ptr(blocks), N, _ptr(y), _stream(stream)),
           "gq_q4k_gemv")
    return y


def gq_bf16_gemv(x: torch.Tensor, w: torch.Tensor, y=None, stream=None):
    """Plain bf16 GEMV (the 16-bit comparator), x bf16 [M<=4, K], w bf16 [N, K] -> y bf16 [M, N]."""
    _need(x, "x", (torch.bfloat16,))
    _need(w, "w", (torch.bfloat16,), x.device)
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError(f"w is {tuple(w.shape)}, expected [N, {K}]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check(lib().gq_bf16_gemv(_ptr(x), M, K, _ptr(w), N, _ptr(y), _stream(stream)), "gq_bf16_gemv")
    return y


def gq_stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Read every byte of the contiguous GPU tensor buf once (bandwidth probe);
    sink is a GPU int32/uint32 tensor of at least one element that the kernel may write."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    _need(sink, "sink", (torch.int32, torch.uint32), buf.device)
    nbytes = buf.numel() * buf.element_size()
    _check(lib().gq_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)), "gq_stream_read")


def gq_ingest_group_major(codes: torch.Tensor, scales: torch.Tensor, qweight=None, scales_out=None,
                          stream=None):
    """Group-major codes int8 [n_groups, group, N] + scales fp16 [n_groups, N] ->
    (qweight uint8 [N, K/2], scales fp16 [N, n_groups]), symmetric, K = n_groups * group."""
    _need(codes, "codes", (torch.int8,))
    _need(scales, "scales", (torch.float16,), codes.device)
    ng, g, N = codes.shape
    if tuple(scales.shape) != (ng, N):
        raise ValueError(f"scales is {tuple(scales.shape)}, expected ({ng}, {N})")
    if qweight is None:
        qweight = torch.empty((N, ng * g // 2), dtype=torch.uint8, device=codes.device)
    if scales_out is None:
        scales_out = torch.empty((N, ng), dtype=torch.float16, device=codes.device)
    _check(lib().gq_ingest_group_major(_ptr(codes), _ptr(scales), ng, g, N, _ptr(qweight),
                                       _ptr(scales_out), _stream(stream)), "gq_ingest_group_major")
    return qweight, scales_out
