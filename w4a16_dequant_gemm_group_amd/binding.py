"""Thin ctypes binding of libgq (``include/gq.h``), same names as the C ABI.

The functions here only marshal arguments: they check the dtype, shape,
contiguity and device of every torch tensor they pass (inputs and
caller-supplied outputs alike, all before the first library call), allocate
missing outputs and workspaces with torch (device memory plumbing), and pass
raw pointers plus the current HIP stream to the library.  Every step of the
computation runs in the library's kernels; there is no fallback path.  A
missing ``libgq.so`` raises immediately.
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
    "gq_w4a16_gemm", "gq_w4a16_gemm_workspace_size", "gq_w4a16_gemm_ws", "gq_w4a16_gemm_noalloc",
    "gq_q4k_quantize", "gq_q4k_gemv", "gq_ingest_group_major",
    "gq_w4a16_gemv_f16", "gq_w4a16_gemv_f16_ws", "gq_w4a16_gemm_f16", "gq_w4a16_gemm_f16_ws",
)
# comparators and probes (include/gq_bench.h)
BENCH_EXPORTS = ("gq_bf16_gemv", "gq_stream_read", "gq_probe_mfma_valu", "gq_probe_lds_read")


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
    sz = ctypes.c_size_t
    Q = GqQParams
    L.gq_status_str.restype = ctypes.c_char_p
    L.gq_status_str.argtypes = [c]
    L.gq_version.restype = i32
    L.gq_version.argtypes = []
    mm = [p, i64, i64, p, p, p, i64, Q, p, p]              # x M K qweight scales zeros N p y stream
    mm_ws = [p, i64, i64, p, p, p, i64, Q, p, p, sz, p]    # ... y workspace bytes stream
    sig = {
        "gq_packed_sizes": [i64, i64, Q, ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(i64)],
        "gq_quantize_groups": [p, c, i64, i64, Q, p, p, p, p],
        "gq_pack_int4": [p, i64, i64, i32, p, p],
        "gq_dequantize": [p, p, p, i64, i64, Q, p, c, p],
        "gq_w4a16_gemv": mm,
        "gq_w4a16_gemv_workspace_size": [i64, i64, i64, Q, ctypes.POINTER(sz)],
        "gq_w4a16_gemv_ws": mm_ws,
        "gq_w4a16_gemm": mm,
        "gq_w4a16_gemm_workspace_size": [i64, i64, i64, Q, ctypes.POINTER(sz)],
        "gq_w4a16_gemm_ws": mm_ws,
        "gq_w4a16_gemm_noalloc": mm,
        "gq_q4k_quantize": [p, c, i64, i64, p, p],
        "gq_q4k_gemv": [p, i64, i64, p, i64, p, p],
        "gq_bf16_gemv": [p, i64, i64, p, i64, p, p],
        "gq_ingest_group_major": [p, p, i64, i64, i64, p, p, p],
        "gq_w4a16_gemv_f16": mm,
        "gq_w4a16_gemv_f16_ws": mm_ws,
        "gq_w4a16_gemm_f16": mm,
        "gq_w4a16_gemm_f16_ws": mm_ws,
        "gq_stream_read": [p, i64, p, p],
        "gq_probe_mfma_valu": [i32, i32, i32, p, p, p],
        "gq_probe_lds_read": [i32, i32, i32, p, p, p],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = c
    _lib = L
    return L


def _ok(status: int, where: str) -> None:
    if status != GQ_OK:
        raise GqError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t, name: str, dtypes, shape=None):
    """Type, dtype, shape and contiguity of a tensor the library will touch."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_device(dev, **tensors) -> None:
    """Every given tensor is a GPU tensor on `dev` (checked after all shapes)."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if dev is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _groups(K: int, group_size: int) -> int:
    if group_size <= 0 or K % group_size != 0:
        raise ValueError(f"group_size {group_size} must be positive and divide K={K}")
    return K // group_size


_DT = {torch.float32: GQ_F32, torch.float16: GQ_F16, torch.bfloat16: GQ_BF16}


def qparams(bits: int = 4, group_size: int = 128, symmetric: bool = False) -> GqQParams:
    return GqQParams(int(bits), int(group_size), int(bool(symmetric)))


def gq_version() -> int:
    return int(lib().gq_version())


def gq_packed_sizes(N: int, K: int, bits: int = 4, group_size: int = 128, symmetric: bool = False):
    """(qweight_bytes, scale_bytes, zero_bytes) of an [N, K] weight."""
    q, s, z = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _ok(lib().gq_packed_sizes(N, K, qparams(bits, group_size, symmetric),
                              ctypes.byref(q), ctypes.byref(s), ctypes.byref(z)), "gq_packed_sizes")
    return q.value, s.value, z.value


def gq_quantize_groups(w: torch.Tensor, bits: int = 4, group_size: int = 128,
                       symmetric: bool = False, codes=None, scales=None, zeros=None, stream=None):
    """w [N, K] (bf16/fp16/fp32) -> (codes u8/i8 [N,K], scales fp16 [N,K/G], zeros fp16 or None)."""
    _need(w, "w", tuple(_DT))
    if w.dim() != 2:
        raise ValueError(f"w must be 2-D, got {tuple(w.shape)}")
    N, K = w.shape
    ng = _groups(K, group_size)
    cdt = torch.int8 if symmetric else torch.uint8
    if codes is not None:
        _need(codes, "codes", (cdt,), (N, K))
    if scales is not None:
        _need(scales, "scales", (torch.float16,), (N, ng))
    if zeros is not None:
        if symmetric:
            raise ValueError("zeros must be None for symmetric quantization")
        _need(zeros, "zeros", (torch.float16,), (N, ng))
    _on_device(None, w=w)
    dev = w.device
    _on_device(dev, codes=codes, scales=scales, zeros=zeros)
    if codes is None:
        codes = torch.empty((N, K), dtype=cdt, device=dev)
    if scales is None:
        scales = torch.empty((N, ng), dtype=torch.float16, device=dev)
    if zeros is None and not symmetric:
        zeros = torch.empty((N, ng), dtype=torch.float16, device=dev)
    _ok(lib().gq_quantize_groups(_ptr(w), _DT[w.dtype], N, K, qparams(bits, group_size, symmetric),
                                 _ptr(codes), _ptr(scales), _ptr(zeros), _stream(stream)),
        "gq_quantize_groups")
    return codes, scales, zeros


def gq_pack_int4(codes: torch.Tensor, symmetric: bool = False, qweight=None, stream=None):
    """codes [N, K] -> qweight uint8 [N, K/2] (low nibble = even k)."""
    _need(codes, "codes", (torch.uint8, torch.int8))
    if codes.dim() != 2 or codes.shape[1] % 2:
        raise ValueError(f"codes must be [N, K] with K even, got {tuple(codes.shape)}")
    N, K = codes.shape
    if qweight is not None:
        _need(qweight, "qweight", (torch.uint8,), (N, K // 2))
    _on_device(None, codes=codes)
    _on_device(codes.device, qweight=qweight)
    if qweight is None:
        qweight = torch.empty((N, K // 2), dtype=torch.uint8, device=codes.device)
    _ok(lib().gq_pack_int4(_ptr(codes), N, K, int(bool(symmetric)), _ptr(qweight), _stream(stream)),
        "gq_pack_int4")
    return qweight


def _weights(qweight, scales, zeros, group_size: int, symmetric: bool):
    """Check the packed weight bundle; returns (N, K, n_groups)."""
    _need(qweight, "qweight", (torch.uint8,))
    if qweight.dim() != 2:
        raise ValueError(f"qweight must be [N, K/2], got {tuple(qweight.shape)}")
    N, K = qweight.shape[0], qweight.shape[1] * 2
    ng = _groups(K, group_size)
    _need(scales, "scales", (torch.float16,), (N, ng))
    if symmetric:
        if zeros is not None:
            raise ValueError("zeros must be None for symmetric weights")
    else:
        if zeros is None:
            raise ValueError("asymmetric weights need zeros")
        _need(zeros, "zeros", (torch.float16,), (N, ng))
    return N, K, ng


def gq_dequantize(qweight: torch.Tensor, scales: torch.Tensor, zeros: Optional[torch.Tensor],
                  group_size: int = 128, symmetric: bool = False, out_dtype=torch.float32,
                  out=None, stream=None):
    """Packed INT4 -> W^ [N, K] in out_dtype (fp32 exact; bf16/fp16 nearest-even)."""
    N, K, _ = _weights(qweight, scales, zeros, group_size, symmetric)
    if out is not None:
        _need(out, "out", tuple(_DT), (N, K))
    _on_device(None, qweight=qweight)
    _on_device(qweight.device, scales=scales, zeros=zeros, out=out)
    if out is None:
        if out_dtype not in _DT:
            raise TypeError(f"out_dtype {out_dtype} not in {tuple(_DT)}")
        out = torch.empty((N, K), dtype=out_dtype, device=qweight.device)
    _ok(lib().gq_dequantize(_ptr(qweight), _ptr(scales), _ptr(zeros), N, K,
                            qparams(4, group_size, symmetric), _ptr(out), _DT[out.dtype],
                            _stream(stream)), "gq_dequantize")
    return out


def gq_w4a16_gemv_workspace_size(M: int, K: int, N: int, group_size: int = 128,
                                 symmetric: bool = False) -> int:
    """Bytes of scratch gq_w4a16_gemv_ws / gq_w4a16_gemv_f16_ws can use (0: none)."""
    b = ctypes.c_size_t()
    _ok(lib().gq_w4a16_gemv_workspace_size(M, K, N, qparams(4, group_size, symmetric),
                                           ctypes.byref(b)), "gq_w4a16_gemv_workspace_size")
    return int(b.value)


def gq_w4a16_gemm_workspace_size(M: int, K: int, N: int, group_size: int = 128,
                                 symmetric: bool = False) -> int:
    """Bytes of scratch gq_w4a16_gemm_ws / gq_w4a16_gemm_f16_ws can use (0: none).
    The size depends on the current device's compute-unit count."""
    b = ctypes.c_size_t()
    _ok(lib().gq_w4a16_gemm_workspace_size(M, K, N, qparams(4, group_size, symmetric),
                                           ctypes.byref(b)), "gq_w4a16_gemm_workspace_size")
    return int(b.value)


# workspace sizes of the shapes seen so far, per device: the query is a host
# call into the library, repeated for every matmul otherwise
_ws_sizes = {}


def _workspace_size(gemv: bool, dev, M, K, N, group_size, symmetric) -> int:
    key = (gemv, dev, M, K, N, group_size, bool(symmetric))
    n = _ws_sizes.get(key)
    if n is None:
        size = gq_w4a16_gemv_workspace_size if gemv else gq_w4a16_gemm_workspace_size
        n = _ws_sizes[key] = size(M, K, N, group_size, symmetric)
    return n


def _matmul(name, x, qweight, scales, zeros, group_size, symmetric, y, stream, workspace,
            xdtype, gemv):
    """Shared marshalling of the four fused matmuls.  A workspace the call can use
    comes from `workspace` (a uint8 GPU tensor of at least the queried size) or
    is allocated with torch on the call's stream, so the caching allocator hands
    that memory to other work only after the call's kernels (and, under stream
    capture, from the graph's own pool)."""
    _need(x, "x", (xdtype,))
    if x.dim() != 2:
        raise ValueError(f"x must be [M, K], got {tuple(x.shape)}")
    M, K = x.shape
    _need(qweight, "qweight", (torch.uint8,))
    if qweight.dim() != 2 or qweight.shape[1] * 2 != K:
        raise ValueError(f"qweight {tuple(qweight.shape)} does not match K={K}")
    N, _, _ = _weights(qweight, scales, zeros, group_size, symmetric)
    if gemv and M > 16:
        raise ValueError(f"the GEMV takes M <= 16, got M={M}")
    if y is not None:
        _need(y, "y", (xdtype,), (M, N))
    if workspace is not None:
        _need(workspace, "workspace", (torch.uint8,))
    _on_device(None, x=x)
    _on_device(x.device, qweight=qweight, scales=scales, zeros=zeros, y=y, workspace=workspace)
    need = _workspace_size(gemv, x.device, M, K, N, group_size, symmetric) if M > 0 and N > 0 else 0
    if workspace is not None and workspace.numel() < need:
        raise ValueError(f"workspace has {workspace.numel()} bytes, the call needs {need}")
    if y is None:
        y = torch.empty((M, N), dtype=xdtype, device=x.device)
    if need > 0 and workspace is None:
        if stream is not None and not hasattr(stream, "cuda_stream"):
            raise ValueError("with a raw stream handle the caller passes the workspace "
                             f"({need} bytes) that the call needs")
        if stream is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        else:
            with torch.cuda.stream(stream):
                workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    fn = getattr(lib(), name + "_ws")
    _ok(fn(_ptr(x), M, K, _ptr(qweight), _ptr(scales), _ptr(zeros), N,
           qparams(4, group_size, symmetric), _ptr(y), _ptr(workspace),
           0 if workspace is None else workspace.numel(), _stream(stream)), name + "_ws")
    return y


def gq_w4a16_gemv(x, qweight, scales, zeros, group_size: int = 128, symmetric: bool = False,
                  y=None, stream=None, workspace=None):
    """Fused W4A16 GEMV, x bf16 [M<=16, K] -> y bf16 [M, N] (through gq_w4a16_gemv_ws)."""
    return _matmul("gq_w4a16_gemv", x, qweight, scales, zeros, group_size, symmetric, y, stream,
                   workspace, torch.bfloat16, True)


def gq_w4a16_gemm(x, qweight, scales, zeros, group_size: int = 128, symmetric: bool = False,
                  y=None, stream=None, workspace=None):
    """Fused W4A16 GEMM (bf16 MFMA), x bf16 [M, K] -> y bf16 [M, N] (through gq_w4a16_gemm_ws)."""
    return _matmul("gq_w4a16_gemm", x, qweight, scales, zeros, group_size, symmetric, y, stream,
                   workspace, torch.bfloat16, False)


def gq_w4a16_gemv_f16(x, qweight, scales, zeros, group_size: int = 128, symmetric: bool = False,
                      y=None, stream=None, workspace=None):
    """Fused W4A16 GEMV with fp16 activations, x fp16 [M<=16, K] -> y fp16 [M, N]."""
    return _matmul("gq_w4a16_gemv_f16", x, qweight, scales, zeros, group_size, symmetric, y, stream,
                   workspace, torch.float16, True)


def gq_w4a16_gemm_f16(x, qweight, scales, zeros, group_size: int = 128, symmetric: bool = False,
                      y=None, stream=None, workspace=None):
    """Fused W4A16 GEMM with fp16 activations (fp16 MFMA), x fp16 [M, K] -> y fp16 [M, N]."""
    return _matmul("gq_w4a16_gemm_f16", x, qweight, scales, zeros, group_size, symmetric, y, stream,
                   workspace, torch.float16, False)


def gq_w4a16_plain(name: str, x, qweight, scales, zeros, group_size: int = 128,
                   symmetric: bool = False, y=None, stream=None):
    """One of the entry points without a workspace (gq_w4a16_gemv, gq_w4a16_gemm
    or their _f16 forms), called as it is; for tests of those entry points."""
    xdtype = torch.float16 if name.endswith("_f16") else torch.bfloat16
    _need(x, "x", (xdtype,))
    M, K = x.shape
    N, Kw, _ = _weights(qweight, scales, zeros, group_size, symmetric)
    if Kw != K:
        raise ValueError(f"qweight {tuple(qweight.shape)} does not match K={K}")
    if y is not None:
        _need(y, "y", (xdtype,), (M, N))
    _on_device(None, x=x)
    _on_device(x.device, qweight=qweight, scales=scales, zeros=zeros, y=y)
    if y is None:
        y = torch.empty((M, N), dtype=xdtype, device=x.device)
    _ok(getattr(lib(), name)(_ptr(x), M, K, _ptr(qweight), _ptr(scales), _ptr(zeros), N,
                             qparams(4, group_size, symmetric), _ptr(y), _stream(stream)), name)
    return y


def gq_w4a16_gemm_noalloc(x, qweight, scales, zeros, group_size: int = 128, symmetric: bool = False,
                          y=None, stream=None):
    """gq_w4a16_gemm with its split scratch in the library's fixed device array
    (no allocation by the call; calls that overlap on one GPU race)."""
    return gq_w4a16_plain("gq_w4a16_gemm_noalloc", x, qweight, scales, zeros, group_size, symmetric,
                          y, stream)


def gq_q4k_quantize(w: torch.Tensor, blocks=None, stream=None):
    """w [N, K] (K % 256 == 0) -> blocks uint8 [N, K/256, 144]."""
    _need(w, "w", tuple(_DT))
    if w.dim() != 2 or w.shape[1] % 256:
        raise ValueError(f"w must be [N, K] with K % 256 == 0, got {tuple(w.shape)}")
    N, K = w.shape
    if blocks is not None:
        _need(blocks, "blocks", (torch.uint8,), (N, K // 256, 144))
    _on_device(None, w=w)
    _on_device(w.device, blocks=blocks)
    if blocks is None:
        blocks = torch.empty((N, K // 256, 144), dtype=torch.uint8, device=w.device)
    _ok(lib().gq_q4k_quantize(_ptr(w), _DT[w.dtype], N, K, _ptr(blocks), _stream(stream)),
        "gq_q4k_quantize")
    return blocks


def gq_q4k_gemv(x: torch.Tensor, blocks: torch.Tensor, y=None, stream=None):
    """Fused GEMV over super-block weights, x bf16 [M<=16, K] -> y bf16 [M, N]."""
    _need(x, "x", (torch.bfloat16,))
    if x.dim() != 2:
        raise ValueError(f"x must be [M, K], got {tuple(x.shape)}")
    M, K = x.shape
    if K % 256:
        raise ValueError(f"K={K} must be a multiple of 256")
    _need(blocks, "blocks", (torch.uint8,))
    if blocks.dim() != 3 or blocks.shape[1] * 256 != K or blocks.shape[2] != 144:
        raise ValueError(f"blocks has shape {tuple(blocks.shape)}, expected (N, {K // 256}, 144)")
    N = blocks.shape[0]
    if y is not None:
        _need(y, "y", (torch.bfloat16,), (M, N))
    _on_device(None, x=x)
    _on_device(x.device, blocks=blocks, y=y)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _ok(lib().gq_q4k_gemv(_ptr(x), M, K, _ptr(blocks), N, _ptr(y), _stream(stream)), "gq_q4k_gemv")
    return y


def gq_bf16_gemv(x: torch.Tensor, w: torch.Tensor, y=None, stream=None):
    """Plain bf16 GEMV (the 16-bit comparator), x bf16 [M<=4, K], w bf16 [N, K] -> y bf16 [M, N]."""
    _need(x, "x", (torch.bfloat16,))
    M, K = x.shape
    _need(w, "w", (torch.bfloat16,))
    if w.dim() != 2 or w.shape[1] != K:
        raise ValueError(f"w is {tuple(w.shape)}, expected [N, {K}]")
    N = w.shape[0]
    if y is not None:
        _need(y, "y", (torch.bfloat16,), (M, N))
    _on_device(None, x=x)
    _on_device(x.device, w=w, y=y)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _ok(lib().gq_bf16_gemv(_ptr(x), M, K, _ptr(w), N, _ptr(y), _stream(stream)), "gq_bf16_gemv")
    return y


def gq_stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Read every byte of the contiguous GPU tensor buf once (bandwidth probe);
    sink is a GPU int32/uint32 tensor of at least one element that the kernel may write."""
    if not isinstance(buf, torch.Tensor) or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous tensor")
    _need(sink, "sink", (torch.int32, torch.uint32))
    if sink.numel() < 1:
        raise ValueError("sink needs at least one element")
    _on_device(None, buf=buf)
    _on_device(buf.device, sink=sink)
    nbytes = buf.numel() * buf.element_size()
    _ok(lib().gq_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)), "gq_stream_read")


def gq_probe_mfma_valu(valu: int, iters: int, grid: int, stream=None) -> torch.Tensor:
    """Per-wave loop cycles [grid * 8] (int64, on the current device) of the
    matrix-core / vector-ALU issue probe (include/gq_bench.h)."""
    dev = torch.device("cuda", torch.cuda.current_device())
    cycles = torch.zeros(grid * 8, dtype=torch.int64, device=dev)
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    _ok(lib().gq_probe_mfma_valu(valu, iters, grid, _ptr(cycles), _ptr(sink), _stream(stream)),
        "gq_probe_mfma_valu")
    return cycles


def gq_probe_lds_read(waves: int, iters: int, grid: int, stream=None) -> torch.Tensor:
    """Per-wave loop cycles [grid * waves] (int64, on the current device) of the
    LDS read probe (include/gq_bench.h)."""
    dev = torch.device("cuda", torch.cuda.current_device())
    cycles = torch.zeros(grid * waves, dtype=torch.int64, device=dev)
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    _ok(lib().gq_probe_lds_read(waves, iters, grid, _ptr(cycles), _ptr(sink), _stream(stream)),
        "gq_probe_lds_read")
    return cycles


def gq_ingest_group_major(codes: torch.Tensor, scales: torch.Tensor, qweight=None, scales_out=None,
                          stream=None):
    """Group-major codes int8 [n_groups, group, N] + scales fp16 [n_groups, N] ->
    (qweight uint8 [N, K/2], scales fp16 [N, n_groups]), symmetric, K = n_groups * group."""
    _need(codes, "codes", (torch.int8,))
    if codes.dim() != 3:
        raise ValueError(f"codes must be [n_groups, group, N], got {tuple(codes.shape)}")
    ng, g, N = codes.shape
    _need(scales, "scales", (torch.float16,), (ng, N))
    if qweight is not None:
        _need(qweight, "qweight", (torch.uint8,), (N, ng * g // 2))
    if scales_out is not None:
        _need(scales_out, "scales_out", (torch.float16,), (N, ng))
    _on_device(None, codes=codes)
    _on_device(codes.device, scales=scales, qweight=qweight, scales_out=scales_out)
    if qweight is None:
        qweight = torch.empty((N, ng * g // 2), dtype=torch.uint8, device=codes.device)
    if scales_out is None:
        scales_out = torch.empty((N, ng), dtype=torch.float16, device=codes.device)
    _ok(lib().gq_ingest_group_major(_ptr(codes), _ptr(scales), ng, g, N, _ptr(qweight),
                                    _ptr(scales_out), _stream(stream)), "gq_ingest_group_major")
    return qweight, scales_out
