/*
 * gq_bench.h - comparators and probes exported by libgq beside the quantized
 * path of gq.h.  Nothing here quantizes: these are the 16-bit baseline, the
 * bandwidth ceiling that the 4-bit kernels are measured against, and two
 * issue-rate probes of the GPU facts the kernels are designed around.
 *
 *   [P1] "vLLM 量化与推测解码：怎样减少容量、带宽与串行轮次", section 2: at
 *        decode every weight is read once per token, so the time follows the
 *        weight bytes; a 4-bit weight moves about a quarter of a 16-bit one.
 *   [P2] "量化" chapter S08, section "亲手实现": the unfused path that first
 *        writes the full-precision weight and then multiplies moves more bytes
 *        than the 16-bit model and is slower.  gq_dequantize (gq.h) followed by
 *        gq_bf16_gemv is that path.
 *
 * Conventions are those of gq.h: device pointers, row-major W [N, K] with
 * Y = X W^T, bf16 as uint16_t bits, host-side validation before any launch,
 * asynchronous execution on `stream`, gfx950 only.  No memory is allocated.
 */
#ifndef GQ_BENCH_H_
#define GQ_BENCH_H_

#include <stdint.h>

#include "gq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Plain bf16 GEMV [P1 sec.2; P2 "亲手实现" unfused path], 1 <= M <= 4:
 *   y[m, n] = bf16( sum_k x[m, k] w[n, k] ), fp32 accumulation, output rounded
 *   to nearest even.
 *   x [M, K] bf16, w [N, K] bf16, y [M, N] bf16; K % 8 == 0.
 * x and w must be 16-byte aligned, y 2-byte aligned.  Errors: INVALID_ARG
 * (M outside 0..4, K < 8 or not a multiple of 8, negative N, NULL),
 * UNSUPPORTED (N * K * 2 >= 2^31 bytes, M * K above the 32768 activations the
 * kernel stages in LDS after rounding K up to a multiple of 2048, device),
 * MISALIGNED. */
gq_status gq_bf16_gemv(const uint16_t* x, int64_t M, int64_t K, const uint16_t* w, int64_t N,
                       uint16_t* y, void* stream);

/* HBM stream read: reads every 16-byte word of buf[0, bytes) once with
 * nontemporal loads.  The words are folded into a value that is stored to
 * *sink only in the rare case that it equals a fixed constant, so *sink must be
 * writable but its content is meaningless.  Timing this call over a buffer much
 * larger than the 256 MB Infinity Cache gives the read bandwidth a kernel can
 * reach.  bytes % 16 == 0, 0 <= bytes <= 2^38.  Errors: INVALID_ARG,
 * MISALIGNED (buf not 16-byte aligned, sink not 4-byte aligned), UNSUPPORTED
 * (device). */
gq_status gq_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

/* Issue-rate probe of the matrix cores and the vector ALU: `grid` workgroups of
 * 512 threads (two waves per SIMD) each run `iters` iterations in which every
 * wave issues 8 independent v_mfma_f32_32x32x16_bf16, each followed by
 * valu / 8 independent fp32 FMAs; wave w of workgroup g writes its loop's
 * s_memtime cycle count to cycles[8 g + w].  valu in {0, 32, 64, 128};
 * 1 <= iters <= 2^20, 1 <= grid <= 65536.  cycles (8-byte aligned, 8 grid
 * entries) and sink (4-byte aligned, never read, written only in a rare case)
 * are device pointers.  Errors: INVALID_ARG, MISALIGNED, UNSUPPORTED (device). */
gq_status gq_probe_mfma_valu(int32_t valu, int32_t iters, int32_t grid, uint64_t* cycles, float* sink,
                             void* stream);

/* LDS read probe: `grid` workgroups of `waves` waves (1..16) each fill a
 * 64 KiB LDS buffer and then run `iters` iterations of 16 independent
 * conflict-free 16-byte reads per lane; wave w of workgroup g writes its
 * loop's s_memtime cycle count to cycles[waves g + w].  LDS bytes per clock
 * of a compute unit = waves * iters * 16 KiB / cycles when one workgroup
 * runs per compute unit.  Limits and errors as gq_probe_mfma_valu. */
gq_status gq_probe_lds_read(int32_t waves, int32_t iters, int32_t grid, uint64_t* cycles, float* sink,
                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQ_BENCH_H_ */
