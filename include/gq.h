/*
 * gq.h - C ABI of libgq: group-wise low-bit weight quantization and the fused
 * W4A16 matmul for AMD MI355X (gfx950).
 *
 * The operations follow these pages (cited by title and section):
 *   [P1] "vLLM 量化与推测解码：怎样减少容量、带宽与串行轮次", section 1
 *        "从实数到有限编码" (affine map q = clamp(round(x/s)+z, qmin, qmax),
 *        x^ = s(q-z); min-max scale and zero; per-group quantization whose
 *        inputs are a float tensor, bits and a group size and whose outputs are
 *        codes plus a (scale, zero) per group) and section 2 (Y = X W^T; weight
 *        bytes = N b/8 + metadata; the fused W4A16 kernel that reads packed
 *        INT4 and group scales, dequantizes on chip, multiplies bf16/fp16
 *        activations with a wider accumulator and never stores the expanded
 *        weight; checkpoints carry packed qweight + scales + zeros + group_size).
 *   [P2] "量化" chapter S08, sections "核心思路" (symmetric group quantizer with
 *        an fp16 scale), "工作原理" (figure: group scales, the 256-weight
 *        super-block with 6-bit sub-block scales/mins, fused dequantization)
 *        and "亲手实现" (group-by-group fused matmul).
 *   [P3] "量化：为何加速推理与精度权衡", sections "直接答案" (affine map and the
 *        bound |x - x^| <= scale/2) and "深入原理" (exact zero).
 *
 * Conventions for every entry point
 *   - Pointers are device pointers (HIP global memory) unless marked "host".
 *     The caller owns every buffer.  libgq allocates nothing, never
 *     synchronizes and keeps no state beyond a per-device architecture and
 *     compute-unit check and a per-process launch-id counter.  Scratch that a
 *     faster kernel can use (split-K partial sums) is passed in by the caller
 *     through the *_ws entry points, sized by the *_workspace_size queries;
 *     the entry points without a workspace run kernels that need none.
 *   - All matrices are dense, row-major, contiguous.  W is [N, K] = out x in,
 *     so Y = X W^T [P1 sec.2]; groups run along K (the reduction axis).
 *   - fp16 / bf16 values are passed as uint16_t bit patterns.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Arguments are
 *     validated on the host before anything is enqueued; on a validation error
 *     nothing is launched and no output is written.  On success the work is
 *     enqueued asynchronously and the call returns GQ_OK; kernel faults surface
 *     on the stream as usual.  A failed launch returns GQ_ERR_HIP and leaves the
 *     outputs undefined.
 *   - Calls are thread-safe; calls on one stream run in order.  A workspace
 *     belongs to one call at a time: calls whose kernels may overlap (on
 *     different streams, or replayed graphs on different streams) must not
 *     share one.
 *   - Only gfx950 devices are accepted (GQ_ERR_UNSUPPORTED otherwise).
 *
 * Storage contract (the readings of the pages used throughout)
 *   - round() is round-half-to-even.
 *   - asymmetric b-bit: codes 0..2^b-1; per group lo = min(min(g), 0),
 *     hi = max(max(g), 0); s = (hi - lo)/(2^b - 1), or 1.0 when hi == lo.
 *   - symmetric b-bit: codes -2^(b-1)..2^(b-1)-1; s = max|g| / (2^(b-1)-1),
 *     or 1.0 when the group is all zero.
 *   - The scale is rounded to fp16 first (nearest-even, saturated to
 *     [2^-24, 65504]); zero point z = clamp(round(-lo/S)) and codes
 *     q = clamp(round(x/S) + z) are computed from that stored S, in binary64.
 *   - zeros are the integer zero points stored as fp16 (exact).
 *   - Packed INT4: qweight[N][K/2]; byte j of a row holds k=2j in bits 0-3
 *     and k=2j+1 in bits 4-7.  Symmetric codes are stored as q+8.
 *   - x^ = S (q - z); symmetric: x^ = S (nibble - 8).
 */
#ifndef GQ_H_
#define GQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GQ_OK = 0,
  GQ_ERR_INVALID_ARG = 1, /* shape/pointer/parameter violates the contract   */
  GQ_ERR_UNSUPPORTED = 2, /* valid request this build does not implement, or
                             a device that is not gfx950                      */
  GQ_ERR_MISALIGNED = 3,  /* a pointer that must be 16-byte aligned is not   */
  GQ_ERR_HIP = 4          /* the HIP runtime reported an error               */
} gq_status;

typedef enum { GQ_F32 = 0, GQ_F16 = 1, GQ_BF16 = 2 } gq_dtype;

/* Quantization parameters [P1 sec.1: bits and group size; symmetric or
 * asymmetric (zero point)].  group_size must divide K; GPU kernels need
 * group_size % 32 == 0. */
typedef struct {
  int32_t bits;       /* 2..8 for quantize; 4 for everything packed */
  int32_t group_size; /* elements per group along K                 */
  int32_t symmetric;  /* 0: asymmetric (scale + zero), 1: symmetric */
} gq_qparams;

/* Human-readable name of a status code (static string). */
const char* gq_status_str(gq_status s);

/* Library ABI version (major*10000 + minor*100 + patch). */
int32_t gq_version(void);

/* Byte sizes of the stored form of an [N, K] weight [P1 sec.2: payload
 * N*K*bits/8 plus a 2-byte scale and (asymmetric) a 2-byte zero per group].
 * Host only; any output pointer may be NULL.  Errors: INVALID_ARG for
 * N, K < 1, bits outside 2..8, or group_size < 1 or not dividing K. */
gq_status gq_packed_sizes(int64_t N, int64_t K, gq_qparams p, int64_t* qweight_bytes,
                          int64_t* scale_bytes, int64_t* zero_bytes);

/* Group-wise affine quantization [P1 sec.1 equations and per-group listing;
 * P2 "核心思路" symmetric quantizer; P3 "直接答案"].
 *   w      [N, K] of w_dtype (GQ_BF16, GQ_F16 or GQ_F32), finite values
 *   codes  [N, K] bytes: uint8 0..2^b-1 (asymmetric) or int8 (symmetric)
 *   scales [N, K/group_size] fp16
 *   zeros  [N, K/group_size] fp16, or NULL exactly when p.symmetric
 * Bit-exact with the storage contract above.  Errors: INVALID_ARG (shape,
 * bits outside 2..8, group_size % 32 != 0 or not dividing K, zeros NULL-ness
 * not matching symmetric, NULL buffers), UNSUPPORTED (device). */
gq_status gq_quantize_groups(const void* w, gq_dtype w_dtype, int64_t N, int64_t K, gq_qparams p,
                             void* codes, uint16_t* scales, uint16_t* zeros, void* stream);

/* INT4 nibble packing [P1 sec.1: two INT4 values per byte; sec.4 "packed
 * qweight"].  codes [N, K] (uint8 0..15, or int8 -8..7 when symmetric) ->
 * qweight [N, K/2].  Codes outside the range are masked to 4 bits.
 * Errors: INVALID_ARG (N, K < 1, K odd, NULL), UNSUPPORTED (device). */
gq_status gq_pack_int4(const void* codes, int64_t N, int64_t K, int32_t symmetric, uint8_t* qweight,
                       void* stream);

/* Dequantization x^ = S (q - z) [P1 sec.1; P2 "核心思路" dequantize_group]:
 * the materialized weight that the fused kernels never write.  Used for tests
 * and as the unfused comparison path [P2 "亲手实现", pitfall paragraph].
 *   qweight [N, K/2], scales/zeros [N, K/group_size] (zeros NULL iff symmetric)
 *   w_hat   [N, K] of out_dtype: GQ_F32 exact, GQ_BF16/GQ_F16 nearest-even.
 * Errors: INVALID_ARG, UNSUPPORTED (bits != 4, device). */
gq_status gq_dequantize(const uint8_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                        int64_t N, int64_t K, gq_qparams p, void* w_hat, gq_dtype out_dtype,
                        void* stream);

/* Ingest of another layout into the canonical one [P2 "亲手实现": its fused
 * matmul keeps int8 codes [n_groups, group, N] (K-major, N contiguous) and fp16
 * scales [n_groups, N] from the symmetric quantizer of "核心思路"]:
 *   codes      [n_groups, group, N] int8, 4-bit symmetric codes -8..7
 *   scales     [n_groups, N] fp16
 *   qweight    [N, K/2] symmetric packed form (nibble = code + 8, low nibble =
 *              even k), K = n_groups * group; 16-byte aligned
 *   scales_out [N, n_groups] fp16
 * The result serves gq_w4a16_gemv / gq_w4a16_gemm with symmetric = 1 and
 * group_size = group.  Codes outside -8..7 are masked to 4 bits, as in
 * gq_pack_int4.  Errors: INVALID_ARG (group % 32 != 0, shapes, NULL),
 * MISALIGNED, UNSUPPORTED (device). */
gq_status gq_ingest_group_major(const int8_t* codes, const uint16_t* scales, int64_t n_groups,
                                int64_t group, int64_t N, uint8_t* qweight, uint16_t* scales_out,
                                void* stream);

/* Fused W4A16 GEMV for decode, 1 <= M <= 16 [P1 sec.2 fused-kernel paragraph;
 * P2 "工作原理" figure right panel and "亲手实现"; P3 "直接答案" (decode is
 * memory-bound)]:
 *   y[m, n] = bf16( sum_g S[n,g] * sum_{k in g} x[m,k] * (q[n,k] - z[n,g]) )
 * with fp32 accumulation, output rounded to nearest-even bf16.
 *   x [M, K] bf16, qweight [N, K/2], scales/zeros [N, K/group_size] fp16
 *   (zeros NULL iff symmetric), y [M, N] bf16.
 * x, qweight and y must be 16-byte aligned.  Errors: INVALID_ARG (M outside
 * 1..16, shapes, group_size % 32, zeros NULL-ness), UNSUPPORTED (bits != 4,
 * device), MISALIGNED. */
gq_status gq_w4a16_gemv(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                        const uint16_t* scales, const uint16_t* zeros, int64_t N, gq_qparams p,
                        uint16_t* y, void* stream);

/* Scratch (bytes) that gq_w4a16_gemv_ws can use for these arguments; 0 when no
 * kernel for them would use any.  1 <= M <= 4 runs a streaming kernel that needs none
 * while x fits its LDS stage (K <= 65536, 34816, 22528, 16384 for M = 1, 2,
 * 3, 4).  5 <= M <= 16 (and M = 4 beyond that K) runs a matrix-core kernel
 * that needs none either when the group size is 32, 64, 128, 256 or a
 * multiple of 512 and K is a multiple of 512: any such K for M <= 8 (x staged
 * in chunks of up to 8192 columns), K <= 4096 for M > 8.  Otherwise, with
 * 4 <= M <= 16, group_size 32, 64 or a multiple of 128 and K % 256 == 0, a
 * workspace lets the GEMV run on the matrix cores split along K into
 * 1024-wide slices with fp32 partial sums per slice: ceil(K / 1024) * M * N * 4
 * bytes (without one it runs a slower per-row dot-product kernel).  The same
 * size serves gq_w4a16_gemv_f16_ws.  Host only.  Errors: INVALID_ARG (M
 * outside 0..16, shapes, group_size, a NULL `bytes`), UNSUPPORTED (bits != 4). */
gq_status gq_w4a16_gemv_workspace_size(int64_t M, int64_t K, int64_t N, gq_qparams p,
                                       size_t* bytes);

/* gq_w4a16_gemv with caller-provided scratch (also usable under stream
 * capture: the call allocates nothing).  workspace: device memory of at least
 * gq_w4a16_gemv_workspace_size() bytes, 16-byte aligned (NULL allowed when
 * that size is 0); this call's kernels on `stream` write it, and nothing else
 * may use it until they complete.  Same result bits as gq_w4a16_gemv up to the
 * summation order of the kernel that runs.  Errors: those of gq_w4a16_gemv,
 * and INVALID_ARG / MISALIGNED for a needed workspace that is NULL, smaller
 * than required or not 16-byte aligned. */
gq_status gq_w4a16_gemv_ws(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                           const uint16_t* scales, const uint16_t* zeros, int64_t N,
                           gq_qparams p, uint16_t* y, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Fused W4A16 GEMM for prefill-sized M (any M >= 1, built for M >= 64) on
 * bf16 MFMA [P1 sec.2; P3 "面试官追问" (weight-only quantization keeps the
 * FLOPs; prefill is compute-bound)].  Same arithmetic, arguments, layout and
 * errors as gq_w4a16_gemv except the M range; additionally UNSUPPORTED for
 * K > 2^22.  The dequantized weight enters the bf16 MFMA as the exact integer
 * q - z and the group scale is applied in fp32, so no weight is rounded.
 * Without a workspace every output tile is computed by one workgroup. */
gq_status gq_w4a16_gemm(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                        const uint16_t* scales, const uint16_t* zeros, int64_t N, gq_qparams p,
                        uint16_t* y, void* stream);

/* Scratch (bytes) that gq_w4a16_gemm_ws can use: when the 256 x 256 output
 * tiles of the last round fill at most half of the GPU's compute units (all
 * tiles when there are at most half as many tiles as compute units), each of
 * those tiles is split along K over two workgroups (each half keeps whole
 * groups and at least two of them), which hand fp32 partial sums over through
 * the workspace: per split tile 16 bytes of handshake words plus a 256 x 256
 * fp32 tile (262144 bytes), the words first and padded to 256 bytes.  0 when
 * nothing would be split (and for K % 64 != 0 or group sizes other than 64,
 * 128 and multiples of 256).  Queries the current device's compute-unit count
 * when a device is present (256 otherwise).  The same size serves
 * gq_w4a16_gemm_f16_ws.  Errors: INVALID_ARG (shapes, group_size, a NULL
 * `bytes`), UNSUPPORTED (bits != 4, K > 2^22). */
gq_status gq_w4a16_gemm_workspace_size(int64_t M, int64_t K, int64_t N, gq_qparams p,
                                       size_t* bytes);

/* gq_w4a16_gemm with caller-provided scratch for the split tiles above.  The
 * workspace needs no initial content (the two workgroups of a split tile tell
 * this call's handshake words from stale ones by a per-call 64-bit id, and the
 * second clears them); it must not be used by other work until this call's
 * kernels complete.  The sum of a split tile does not depend on which half
 * finishes first.  Should a tile's second half wait for the first beyond a
 * bound (about a second; only a lost workgroup could cause it), that tile is
 * written as NaN rather than left wrong.  Errors: those of gq_w4a16_gemm, and
 * INVALID_ARG / MISALIGNED for a needed workspace that is NULL, smaller than
 * gq_w4a16_gemm_workspace_size() or not 16-byte aligned. */
gq_status gq_w4a16_gemm_ws(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                           const uint16_t* scales, const uint16_t* zeros, int64_t N,
                           gq_qparams p, uint16_t* y, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Bytes of the fixed device scratch behind gq_w4a16_gemm_noalloc: the split
 * of the last round on a GPU of up to 256 compute units (at most 128 split
 * tiles: 2048 bytes of handshake words and 128 partial tiles of 262144 bytes),
 * rounded up to 32 MiB + 4 KiB. */
#define GQ_NOALLOC_SCRATCH_BYTES ((size_t)(32u << 20) + 4096u)

/* gq_w4a16_gemm for callers that cannot allocate device memory (code under
 * stream capture, tight serving loops, harnesses that forbid allocation): the
 * same kernels and result as gq_w4a16_gemm_ws, with the split scratch taken
 * from a fixed array of GQ_NOALLOC_SCRATCH_BYTES in device memory that the
 * library holds per GPU until the process ends (its address is looked up once
 * per device, on the first call there).  The call allocates nothing.  Every
 * call on a GPU shares that GPU's array: calls whose kernels may overlap on
 * one GPU (different streams, concurrent graph replays) race and must not be
 * made.  The array keeps the last call's content; nothing in it needs to be
 * zero (the handshake tells stale words from this call's).  Errors: those of
 * gq_w4a16_gemm; UNSUPPORTED when the split would need more than
 * GQ_NOALLOC_SCRATCH_BYTES (not on a 256-CU gfx950); HIP when the array's
 * address cannot be looked up. */
gq_status gq_w4a16_gemm_noalloc(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                                const uint16_t* scales, const uint16_t* zeros, int64_t N,
                                gq_qparams p, uint16_t* y, void* stream);

/* The fused matmuls with fp16 activations and fp16 output [P1 sec.2: the
 * fused kernel multiplies BF16/FP16 activations]: the same product as
 * gq_w4a16_gemv / gq_w4a16_gemm, x [M, K] fp16 and y [M, N] fp16 (rounded to
 * nearest even; overflow gives +-inf), fp32 accumulation, with the same
 * shapes, kernels (fp16 MFMA and fp16 dot products, the nibble taken as the
 * exact fp16 1024 + q), workspaces and errors as the bf16 entry points. */
gq_status gq_w4a16_gemv_f16(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                            const uint16_t* scales, const uint16_t* zeros, int64_t N,
                            gq_qparams p, uint16_t* y, void* stream);
gq_status gq_w4a16_gemv_f16_ws(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                               const uint16_t* scales, const uint16_t* zeros, int64_t N,
                               gq_qparams p, uint16_t* y, void* workspace, size_t workspace_bytes,
                               void* stream);
gq_status gq_w4a16_gemm_f16(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                            const uint16_t* scales, const uint16_t* zeros, int64_t N,
                            gq_qparams p, uint16_t* y, void* stream);
gq_status gq_w4a16_gemm_f16_ws(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                               const uint16_t* scales, const uint16_t* zeros, int64_t N,
                               gq_qparams p, uint16_t* y, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Nested 4-bit super-block format [P2 "工作原理" figure, middle panel: 256
 * weights = 8 sub-blocks of 32, 6-bit scale and 6-bit min per sub-block, fp16
 * scale-of-scales d and min-of-mins dmin per super-block, 4.5 bits/weight].
 * Per sub-block j: lo = min(min,0), hi = max(max,0), s_j = (hi-lo)/15 (0 if
 * equal), m_j = 0 - lo (+0 when lo = 0); d = fp16(max_j s_j / 63),
 * dmin = fp16(max_j m_j / 63), a zero d or dmin stored as +0 (0x0000);
 * sc_j = clamp(round(s_j/d), 0, 63), mn_j = clamp(round(m_j/dmin), 0, 63)
 * (0 when d or dmin is 0); q = clamp(round((x + dmin mn_j)/(d sc_j)), 0, 15)
 * (0 when d sc_j = 0); x^ = d sc_j q - dmin mn_j.  All in binary64.
 * Block bytes (144): [0] d fp16, [2] dmin fp16, [4] sc_0..7 as a 48-bit
 * little-endian stream (6 bits each), [10] mn_0..7 likewise, [16] 128 bytes of
 * nibbles, sub-block j at 16+16j, low nibble = even k.
 *   w [N, K] (K % 256 == 0) -> blocks [N, K/256, 144].
 * Errors: INVALID_ARG, UNSUPPORTED (device). */
gq_status gq_q4k_quantize(const void* w, gq_dtype w_dtype, int64_t N, int64_t K, uint8_t* blocks,
                          void* stream);

/* Fused GEMV over the super-block format, 1 <= M <= 16:
 *   y[m, n] = bf16( sum_j d sc_j sum_k x q - dmin mn_j sum_k x ), fp32 accumulation.
 *   x [M, K] bf16, blocks [N, K/256, 144], y [M, N] bf16.
 * x, blocks and y must be 16-byte aligned.  Errors: INVALID_ARG, MISALIGNED,
 * UNSUPPORTED (device). */
gq_status gq_q4k_gemv(const uint16_t* x, int64_t M, int64_t K, const uint8_t* blocks, int64_t N,
                      uint16_t* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQ_H_ */
