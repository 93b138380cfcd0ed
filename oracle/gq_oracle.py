"""CPU oracle for group-wise INT4 weight quantization and the W4A16 matmul.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, obviously-correct
reference that the GPU library is checked against.  Only the tests, the smoke
check and the benchmark's CPU-baseline leg may import it; the product path
(the C-ABI library and its Python binding) never does, and this module imports
nothing from the product path.

Everything is numpy in float64 (the page-1 and page-3 listings compute in
Python floats, i.e. binary64).  Stored scales are binary16, stored activations
and outputs bf16; both are carried here as ``uint16`` bit patterns.

Sources (the pages' titles; sections / equations named in each docstring):

* [P1] "vLLM 量化与推测解码：怎样减少容量、带宽与串行轮次"
  (liujiyu20000308.github.io) - section 1 "从实数到有限编码" (affine map,
  min-max scale/zero, per-tensor and per-group quantization), section 2
  (Y = X W^T, weight bytes, the fused W4A16 kernel principle, byte examples).
* [P2] "量化" chapter S08 (llminference.xinbetween.com) - "核心思路"
  (symmetric group quantizer, effective bits), "工作原理" figure (group
  scales, the Q4_K super-block, fused dequantization), "亲手实现" (group-by-group
  fused matmul with a float64 accumulator).
* [P3] "量化：为何加速推理与精度权衡" (inference-learning-path) - "直接答案"
  (affine map, error bound scale/2), "深入原理" (exact zero), "代码" (worked
  example [-0.9, -0.2, 0.1, 0.5, 3.0] at 4 bits).

Readings taken where the pages are open (each also listed in the design notes):

R1  round() is round-half-to-even (numpy.rint), as Python's round and
    numpy.round both are in the pages' listings.
R2  The asymmetric range always contains 0: lo = min(min(g), 0),
    hi = max(max(g), 0) [P1 section 1 listing]; needed for [P3]'s exact zero.
R3  A degenerate range (hi == lo, or max|g| == 0) uses scale 1.0 [P1 listing].
R4  The scale is rounded to fp16 *first* and zero point and codes are derived
    from that stored scale, so the [P3] bound |x - x^| <= scale/2 holds for the
    scale actually used by dequantization.  The fp16 rounding is nearest-even
    and saturates to the finite positive fp16 range [2^-24, 65504].
R5  The zero point is an integer stored as fp16 (exact); symmetric codes
    are stored offset-binary (q + 8) in the nibble.
R6  Packing: qweight is [N, K/2] bytes, byte j of row n holds code k=2j in
    bits 0-3 and k=2j+1 in bits 4-7 ([P1] only says two INT4 per byte).
R7  The super-block format's own quantizer (the pages give only its sizes):
    per 32-wide sub-block an unsigned 4-bit code with a zero-inclusive min,
    x^ = d*sc*q - dmin*mn, 6-bit sc/mn by round-to-nearest against fp16 d/dmin
    taken from the block maxima / 63.  A zero d or dmin is stored as +0
    (bits 0x0000): the sub-block min is m_j = 0 - lo_j, which is +0 when lo_j
    is 0, and a zero scale rounds to +0.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# Number formats.  Library conversions are used as single steps and are pinned
# by the tests (numpy's float64 -> float16 cast is correctly rounded).
# ----------------------------------------------------------------------------

FP16_MAX = 65504.0
FP16_MIN_SUB = 2.0 ** -24


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 values (exact widening)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    """binary16 bit patterns -> float64 values (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f64_to_f16_bits(v: np.ndarray) -> np.ndarray:
    """float64 -> binary16 bits, round to nearest even (one rounding)."""
    with np.errstate(over="ignore"):
        return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def scale_to_f16(v: np.ndarray) -> np.ndarray:
    """Reading R4: a positive scale rounded to fp16, saturated to [2^-24, 65504].

    Zero stays zero (only the super-block format can produce a zero scale)."""
    v = np.asarray(v, dtype=np.float64)
    h = f16_to_f64(f64_to_f16_bits(v))
    h = np.where(np.isinf(h), FP16_MAX, h)
    h = np.where((v > 0) & (h == 0), FP16_MIN_SUB, h)
    return np.where(v > 0, h, 0.0)                     # +0.0, never -0.0


def f32_exact_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float64 values that are exact in float32 -> bf16 bits, nearest-even.

    The float32 bit pattern u rounds to its top 16 bits by adding 0x7FFF plus the
    lowest kept bit (ties go to the even neighbour)."""
    v = np.asarray(v, dtype=np.float64)
    f = v.astype(np.float32)
    if not np.array_equal(f.astype(np.float64), v, equal_nan=True):
        raise ValueError("value not exactly representable in float32")
    u = f.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------
# Group-wise affine quantization [P1 sec.1 eq. q=clamp(round(x/s)+z), x^=s(q-z);
# min-max s=(xmax-xmin)/(qmax-qmin), z=round(qmin-xmin/s)], [P2 symmetric
# quantize_group], [P3 direct answer].
# ----------------------------------------------------------------------------

def code_range(bits: int, symmetric: bool):
    """(qmin, qmax) of the integer codes: unsigned 0..2^b-1 [P1 sec.1], or
    symmetric -(2^(b-1))..2^(b-1)-1 with scale from 2^(b-1)-1 [P2]."""
    if symmetric:
        return -(2 ** (bits - 1)), 2 ** (bits - 1) - 1
    return 0, 2 ** bits - 1


def quantize_groups(w: np.ndarray, bits: int, group_size: int, symmetric: bool,
                    fp16_scale: bool = True):
    """Quantize each row of ``w`` [N, K] in groups of ``group_size`` along K.

    Returns ``(codes int64 [N,K], scales f64 [N,ng], zeros f64 [N,ng] or None)``.
    The last group may be shorter than ``group_size`` ([P1] listing allows it).
    ``fp16_scale=False`` keeps the binary64 scale (the [P1]/[P3] listings have no
    fp16 storage); the library contract is ``fp16_scale=True`` (R4).
    """
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    qmin, qmax = code_range(bits, symmetric)
    starts = list(range(0, K, group_size))
    codes = np.zeros((N, K), dtype=np.int64)
    scales = np.zeros((N, len(starts)))
    zeros = None if symmetric else np.zeros((N, len(starts)))
    for gi, a in enumerate(starts):
        g = w[:, a:a + group_size]
        if symmetric:
            amax = np.abs(g).max(axis=1)
            s = np.where(amax > 0, amax / qmax, 1.0)                  # R3
            S = scale_to_f16(s) if fp16_scale else s
            q = np.clip(np.rint(g / S[:, None]), qmin, qmax)
        else:
            lo = np.minimum(g.min(axis=1), 0.0)                       # R2
            hi = np.maximum(g.max(axis=1), 0.0)
            s = np.where(hi != lo, (hi - lo) / (qmax - qmin), 1.0)    # R3
            S = scale_to_f16(s) if fp16_scale else s                  # R4
            z = np.clip(np.rint(qmin - lo / S), qmin, qmax)
            q = np.clip(np.rint(g / S[:, None]) + z[:, None], qmin, qmax)
            zeros[:, gi] = z
        scales[:, gi] = S
        codes[:, a:a + group_size] = q.astype(np.int64)
    return codes, scales, zeros


def dequantize_codes(codes, scales, zeros, group_size: int):
    """x^ = s (q - z) per group (z = 0 when symmetric) [P1 sec.1; P2 dequantize]."""
    codes = np.asarray(codes, dtype=np.float64)
    N, K = codes.shape
    out = np.empty((N, K))
    for gi, a in enumerate(range(0, K, group_size)):
        z = 0.0 if zeros is None else zeros[:, gi][:, None]
        out[:, a:a + group_size] = scales[:, gi][:, None] * (codes[:, a:a + group_size] - z)
    return out


# ----------------------------------------------------------------------------
# INT4 nibble packing (R5, R6) [P1 sec.1 "two INT4 values per byte"].
# ----------------------------------------------------------------------------

def pack_int4(codes: np.ndarray, symmetric: bool) -> np.ndarray:
    """codes [N,K] (0..15, or -8..7 when symmetric) -> qweight uint8 [N, K/2]."""
    c = np.asarray(codes, dtype=np.int64)
    nib = c + 8 if symmetric else c
    if nib.min(initial=0) < 0 or nib.max(initial=0) > 15:
        raise ValueError("code out of the 4-bit range")
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def unpack_int4(qweight: np.ndarray, symmetric: bool) -> np.ndarray:
    """Inverse of pack_int4."""
    q = np.asarray(qweight, dtype=np.int64)
    N, H = q.shape
    out = np.empty((N, 2 * H), dtype=np.int64)
    out[:, 0::2] = q & 15
    out[:, 1::2] = q >> 4
    return out - 8 if symmetric else out


def dequantize_packed(qweight, scales_bits, zeros_bits, group_size: int, symmetric: bool):
    """Packed 4-bit weight + fp16 scales (+ fp16 zeros) -> exact float64 W^."""
    codes = unpack_int4(qweight, symmetric)
    s = f16_to_f64(scales_bits)
    z = None if symmetric else f16_to_f64(zeros_bits)
    return dequantize_codes(codes, s, z, group_size)


# ----------------------------------------------------------------------------
# Byte accounting [P1 sec.2: B_weight = N_param*b/8 + B_meta; 2-byte scale and
# 2-byte zero per group]; [P2 "4-bit is never 4 bits"].
# ----------------------------------------------------------------------------

def packed_sizes(n: int, k: int, group_size: int, symmetric: bool, bits: int = 4):
    """(qweight bytes, scale bytes, zero bytes) for an [n, k] matrix."""
    ng = -(-k // group_size)
    return n * k * bits // 8, 2 * n * ng, 0 if symmetric else 2 * n * ng


# ----------------------------------------------------------------------------
# Matmul [P1 sec.2 Y = X W^T], fused group-by-group with a float64 accumulator
# [P2 "亲手实现" fused_matmul: out += x[:, group] @ dequant(group)].
# ----------------------------------------------------------------------------

def matmul_groupwise(x: np.ndarray, w_hat: np.ndarray, group_size: int) -> np.ndarray:
    """Y[m, n] = sum over groups g of x[m, g] . w_hat[n, g], accumulated in float64
    one group at a time.  ``x`` [M, K] and ``w_hat`` [N, K] are float64."""
    x = np.asarray(x, dtype=np.float64)
    w_hat = np.asarray(w_hat, dtype=np.float64)
    M, K = x.shape
    out = np.zeros((M, w_hat.shape[0]))
    for a in range(0, K, group_size):
        out += x[:, a:a + group_size] @ w_hat[:, a:a + group_size].T
    return out


def w4a16_reference(x_bits, qweight, scales_bits, zeros_bits, group_size: int,
                    symmetric: bool) -> np.ndarray:
    """Exact-operand float64 reference of the fused W4A16 product for bf16 x."""
    w_hat = dequantize_packed(qweight, scales_bits, zeros_bits, group_size, symmetric)
    return matmul_groupwise(bf16_to_f64(x_bits), w_hat, group_size)


def ingest_group_major(codes_gkn, scales_gn_bits):
    """The "量化" chapter's "亲手实现" layout -> the canonical one.

    codes [n_groups, group, N] signed integers (its symmetric quantizer: -8..7 at
    4 bits), scales [n_groups, N] fp16 bits -> (qweight uint8 [N, K/2] with
    offset-binary nibbles, scales [N, n_groups] fp16 bits), K = n_groups * group.
    Row n of the weight is column n of every group's [group, N] slab."""
    c = np.asarray(codes_gkn, dtype=np.int64)
    ng, g, n = c.shape
    codes_nk = c.reshape(ng * g, n).T
    return pack_int4(codes_nk, True), np.ascontiguousarray(np.asarray(scales_gn_bits, dtype=np.uint16).T)


def quantize_to_storage(w_bits, bits, group_size, symmetric):
    """bf16 weight -> (codes, fp16 scale bits, fp16 zero bits or None) per R1-R5."""
    codes, s, z = quantize_groups(bf16_to_f64(w_bits), bits, group_size, symmetric)
    return codes, f64_to_f16_bits(s), (None if z is None else f64_to_f16_bits(z))


# ----------------------------------------------------------------------------
# Nested super-block 4-bit format [P2 "工作原理" figure, middle panel: 256 weights
# = 8 sub-blocks of 32; each sub-block a 6-bit scale and 6-bit min; each
# super-block an fp16 scale-of-scales and fp16 min-of-mins; 4.5 bits/weight].
# Its quantizer is reading R7.  Block bytes (144):
#   0: d (fp16)   2: dmin (fp16)   4: sc[0..7] 48-bit little-endian stream
#  10: mn[0..7] likewise           16: 128 bytes of nibbles, sub-block j at 16+16j,
#  low nibble = even k.
# ----------------------------------------------------------------------------

Q4K_BLOCK = 256
Q4K_SUB = 32
Q4K_BYTES = 144


def q4k_quantize(w: np.ndarray):
    """w [N, K] (K % 256 == 0) -> dict of per-block fields (float64 / int64)."""
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    nb = K // Q4K_BLOCK
    sub = w.reshape(N, nb, 8, Q4K_SUB)
    lo = np.minimum(sub.min(axis=3), 0.0)
    hi = np.maximum(sub.max(axis=3), 0.0)
    s = np.where(hi != lo, (hi - lo) / 15.0, 0.0)      # sub-block step
    m = 0.0 - lo                                        # sub-block min, +0 (never -0) when lo = 0
    d = scale_to_f16(s.max(axis=2) / 63.0)              # fp16 scale of scales
    dmin = scale_to_f16(m.max(axis=2) / 63.0)           # fp16 min of mins
    with np.errstate(divide="ignore", invalid="ignore"):
        sc = np.where(d[..., None] > 0, np.clip(np.rint(s / d[..., None]), 0, 63), 0)
        mn = np.where(dmin[..., None] > 0, np.clip(np.rint(m / dmin[..., None]), 0, 63), 0)
    S = d[..., None] * sc
    Mn = dmin[..., None] * mn
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(S[..., None] > 0,
                     np.clip(np.rint((sub + Mn[..., None]) / S[..., None]), 0, 15), 0)
    return {"d": d, "dmin": dmin, "sc": sc.astype(np.int64), "mn": mn.astype(np.int64),
            "q": q.astype(np.int64).reshape(N, K)}


def q4k_dequantize_fields(f) -> np.ndarray:
    """x^ = d*sc*q - dmin*mn per sub-block (exact in float64)."""
    N, K = f["q"].shape
    nb = K // Q4K_BLOCK
    q = f["q"].reshape(N, nb, 8, Q4K_SUB).astype(np.float64)
    S = f["d"][..., None] * f["sc"]
    Mn = f["dmin"][..., None] * f["mn"]
    return (S[..., None] * q - Mn[..., None]).reshape(N, K)


def _pack6(vals: np.ndarray) -> np.ndarray:
    """[..., 8] of 6-bit values -> [..., 6] bytes, value j at bits 6j.. of a
    48-bit little-endian integer."""
    acc = np.zeros(vals.shape[:-1], dtype=np.uint64)
    for j in range(8):
        acc |= vals[..., j].astype(np.uint64) << np.uint64(6 * j)
    return np.stack([((acc >> np.uint64(8 * b)) & np.uint64(0xFF)).astype(np.uint8)
                     for b in range(6)], axis=-1)


def _unpack6(b: np.ndarray) -> np.ndarray:
    acc = np.zeros(b.shape[:-1], dtype=np.uint64)
    for i in range(6):
        acc |= b[..., i].astype(np.uint64) << np.uint64(8 * i)
    return np.stack([((acc >> np.uint64(6 * j)) & np.uint64(63)).astype(np.int64)
                     for j in range(8)], axis=-1)


def q4k_encode(f) -> np.ndarray:
    """Fields -> blocks uint8 [N, K/256, 144]."""
    N, K = f["q"].shape
    nb = K // Q4K_BLOCK
    out = np.zeros((N, nb, Q4K_BYTES), dtype=np.uint8)
    out[..., 0:2] = f64_to_f16_bits(f["d"]).view(np.uint8).reshape(N, nb, 2)
    out[..., 2:4] = f64_to_f16_bits(f["dmin"]).view(np.uint8).reshape(N, nb, 2)
    out[..., 4:10] = _pack6(f["sc"])
    out[..., 10:16] = _pack6(f["mn"])
    q = f["q"].reshape(N, nb, Q4K_BLOCK)
    out[..., 16:] = (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)
    return out


def q4k_decode(blocks: np.ndarray):
    """blocks uint8 [N, nb, 144] -> fields (inverse of q4k_encode)."""
    b = np.asarray(blocks, dtype=np.uint8)
    N, nb, _ = b.shape
    d = f16_to_f64(np.ascontiguousarray(b[..., 0:2]).view(np.uint16)[..., 0])
    dmin = f16_to_f64(np.ascontiguousarray(b[..., 2:4]).view(np.uint16)[..., 0])
    q = np.empty((N, nb, Q4K_BLOCK), dtype=np.int64)
    q[..., 0::2] = b[..., 16:] & 15
    q[..., 1::2] = b[..., 16:] >> 4
    return {"d": d, "dmin": dmin, "sc": _unpack6(b[..., 4:10]), "mn": _unpack6(b[..., 10:16]),
            "q": q.reshape(N, nb * Q4K_BLOCK)}


def q4k_reference(x_bits, blocks) -> np.ndarray:
    """float64 Y = X W^T for a super-block-format weight, accumulated one
    32-wide sub-block at a time."""
    w_hat = q4k_dequantize_fields(q4k_decode(blocks))
    return matmul_groupwise(bf16_to_f64(x_bits), w_hat, Q4K_SUB)


# ----------------------------------------------------------------------------
# Error measures used by the parity bar (relative Frobenius error; max error
# against ||x||_inf * ||w^||_inf * sqrt(K) / 64).
# ----------------------------------------------------------------------------

def rel_frobenius(y, y_ref) -> float:
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.linalg.norm(y_ref)
    return float(np.linalg.norm(y - y_ref) / den) if den > 0 else float(np.linalg.norm(y))


def max_err_bound(x64, w_hat64) -> float:
    """1e-2 * max|x| * max|w^| * sqrt(K) / 64: element-wise maxima over the
    whole activation [M, K] and the whole dequantized weight; K the reduction
    length."""
    K = x64.shape[1]
    return 1e-2 * float(np.abs(x64).max()) * float(np.abs(w_hat64).max()) * np.sqrt(K) / 64.0


def bf16_half_ulp(v) -> np.ndarray:
    """Half the spacing of bf16 values at |v| (the rounding error a bf16 output
    can carry on its own); 2^-134 below the normal range."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126.0)
    return np.where(a > 0, 2.0 ** (e - 8), 2.0 ** -134)


def f16_half_ulp(v) -> np.ndarray:
    """Half the spacing of binary16 values at |v|: 11 significant bits, so
    2^(e-11) in [2^e, 2^(e+1)); the subnormal spacing 2^-24 below 2^-14."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -14.0)
    return np.where(a > 0, 2.0 ** (e - 11), 2.0 ** -25)


def within_parity(y, y_ref, x64, w_hat, out: str = "bf16"):
    """The matmul parity bar: relative Frobenius error <= 2e-3 and, element-wise,
    |y - y_ref| <= 1e-2 ||x||_inf ||w^||_inf sqrt(K)/64 plus half an ulp of the
    output format (``out`` = "bf16" or "f16"; the result is stored in that
    format, whose rounding alone may exceed the first term when K is small).
    Returns (ok, rel_f, max_excess_ratio)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    rel = rel_frobenius(y, y_ref)
    half_ulp = {"bf16": bf16_half_ulp, "f16": f16_half_ulp}[out]
    allow = max_err_bound(x64, w_hat) + half_ulp(np.maximum(np.abs(y), np.abs(y_ref)))
    ratio = float((np.abs(y - y_ref) / allow).max()) if y.size else 0.0
    return (rel <= 2e-3 and ratio <= 1.0), rel, ratio


def snr_db(w, w_hat) -> float:
    w = np.asarray(w, dtype=np.float64)
    e = np.asarray(w_hat, dtype=np.float64) - w
    return float(10.0 * np.log10((w * w).sum() / max((e * e).sum(), 1e-300)))
