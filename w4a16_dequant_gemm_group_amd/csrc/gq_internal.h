// Internal declarations shared by the libgq translation units: number-format
// helpers used on the device and the launchers each kernel file provides.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gq.h"
#include "gq_bench.h"

namespace gq {

// ---------------------------------------------------------------------------
// Number formats
// ---------------------------------------------------------------------------

// bf16 bits -> float (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bf16 bits, round to nearest even (inputs here are never NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp16 bits -> float (exact).
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// fp16 bits -> double (exact).
__device__ __forceinline__ double f16_to_f64(uint16_t h) {
  return (double)__builtin_bit_cast(_Float16, h);
}

// double -> fp16 bits with a single round-to-nearest-even step, from the
// binary expansion (no float32 detour, so no double rounding).  Overflow gives
// infinity, underflow zero; NaN stays NaN.
__host__ __device__ inline uint16_t f64_to_f16_rne(double v) {
  uint64_t b;
  __builtin_memcpy(&b, &v, 8);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const int ex = (int)((b >> 52) & 0x7FF);
  const uint64_t man = b & ((1ull << 52) - 1);
  if (ex == 0x7FF) return sign | 0x7C00u | (man ? 0x200u : 0u);
  if (ex == 0) return sign;  // binary64 subnormals are far below fp16's range
  const int e = ex - 1023;
  if (e > 15) return sign | 0x7C00u;
  const uint64_t full = man | (1ull << 52);
  // Keep 11 significant bits for normals; fewer for fp16 subnormals.
  int shift = (e >= -14) ? 42 : 42 + (-14 - e);
  if (shift > 63) return sign;
  uint64_t m = full >> shift;
  const uint64_t rem = full & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (m & 1))) m += 1;
  if (e >= -14) {
    int eb = e + 15;
    if (m == (1ull << 11)) { m >>= 1; eb += 1; }
    if (eb > 30) return sign | 0x7C00u;
    return sign | (uint16_t)(eb << 10) | (uint16_t)(m & 0x3FF);
  }
  return sign | (uint16_t)m;  // m == 0x400 encodes the smallest normal
}

// A positive group scale rounded to fp16 and saturated to [2^-24, 65504];
// zero stays zero.
__host__ __device__ inline uint16_t scale_to_f16(double v) {
  if (!(v > 0.0)) return 0;
  uint16_t h = f64_to_f16_rne(v);
  if ((h & 0x7FFFu) >= 0x7C00u) return 0x7BFFu;
  if (h == 0) return 0x0001u;
  return h;
}

// 16-byte streaming load (read once; the nontemporal hint keeps it from
// displacing reused lines in the caches).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Load one input element of dtype dt as double (exact).
__device__ __forceinline__ double load_elem_f64(const void* p, int64_t i, gq_dtype dt) {
  if (dt == GQ_BF16) return (double)bf16_to_f32(((const uint16_t*)p)[i]);
  if (dt == GQ_F16) return f16_to_f64(((const uint16_t*)p)[i]);
  return (double)((const float*)p)[i];
}

// Compute units of the current device (set by the C ABI's device check).
int num_cus();

// A 64-bit id unique to each launch that needs one (odd, never 0), random
// per process: kernels that hand partial sums between workgroups through
// caller memory of unknown content tell this launch's words from stale ones by it.
uint64_t next_launch_id();

// ---------------------------------------------------------------------------
// Launchers (arguments already validated by the C ABI layer)
// ---------------------------------------------------------------------------

hipError_t launch_quantize_groups(const void* w, gq_dtype dt, int64_t N, int64_t K, int bits,
                                  int G, int symmetric, void* codes, uint16_t* scales,
                                  uint16_t* zeros, hipStream_t s);
hipError_t launch_pack_int4(const void* codes, int64_t N, int64_t K, int symmetric,
                            uint8_t* qweight, hipStream_t s);
hipError_t launch_dequantize(const uint8_t* qweight, const uint16_t* scales,
                             const uint16_t* zeros, int64_t N, int64_t K, int G, int symmetric,
                             void* out, gq_dtype odt, hipStream_t s);
hipError_t launch_ingest_group_major(const int8_t* codes, const uint16_t* scales, int64_t ng,
                                     int64_t group, int64_t N, uint8_t* qweight,
                                     uint16_t* scales_out, hipStream_t s);
// The fused GEMV (1 <= M <= 16).  workspace: caller scratch of at least
// gemv_workspace_bytes(...) bytes for the split-K matrix-core kernel, or NULL
// (the call then runs a kernel that needs none).  xf16: fp16 activations and
// output instead of bf16.
hipError_t launch_w4a16_gemv(const uint16_t* x, int M, int64_t K, const uint8_t* qweight,
                             const uint16_t* scales, const uint16_t* zeros, int64_t N, int G,
                             int symmetric, uint16_t* y, void* workspace, bool xf16, hipStream_t s);
// Whether the persistent streaming GEMV (M = 1..4, no scratch) takes M rows at this K.
bool gemv_stream_supported(int M, int64_t K);
// Small-batch GEMV on the matrix cores with every activation row in LDS and K
// split over the waves of a workgroup (no scratch), where it fits.
bool gemv_mfma_stream_supported(int M, int64_t K, int64_t N, int G);
hipError_t launch_w4a16_gemv_mfma_stream(const uint16_t* x, int M, int64_t K, const uint8_t* qweight,
                                         const uint16_t* scales, const uint16_t* zeros, int64_t N,
                                         int G, int symmetric, uint16_t* y, hipStream_t s,
                                         bool xf16 = false);
// Small-batch GEMV on the matrix cores with x held in registers (4 <= M <=
// 16, K of 512 .. 4096), no scratch.
bool gemv_xreg_supported(int M, int64_t K, int64_t N, int G);
hipError_t launch_w4a16_gemv_xreg(const uint16_t* x, int M, int64_t K, const uint8_t* qweight,
                                  const uint16_t* scales, const uint16_t* zeros, int64_t N, int G,
                                  int symmetric, uint16_t* y, hipStream_t s, bool xf16);
// The same for long K with x streamed from L2 (K > 4096, a multiple of 256).
bool gemv_xs_supported(int M, int64_t K, int64_t N, int G);
hipError_t launch_w4a16_gemv_xs(const uint16_t* x, int M, int64_t K, const uint8_t* qweight,
                                const uint16_t* scales, const uint16_t* zeros, int64_t N, int G,
                                int symmetric, uint16_t* y, hipStream_t s, bool xf16);
// Small-batch GEMV on the matrix cores split along K (4 <= M <= 16), partial
// sums per 1024-wide slice in `workspace`, added by a second kernel.
bool gemv_mfma_supported(int M, int64_t K, int64_t N, int G);
// Scratch the GEMV can use for these arguments (0: no kernel would use any).
size_t gemv_workspace_bytes(int M, int64_t K, int64_t N, int G);
hipError_t launch_w4a16_gemv_mfma(const uint16_t* x, int M, int64_t K, const uint8_t* qweight,
                                  const uint16_t* scales, const uint16_t* zeros, int64_t N, int G,
                                  int symmetric, uint16_t* y, void* workspace, bool xf16,
                                  hipStream_t s);
// The fused GEMM.  workspace: caller scratch of at least gemm_workspace_bytes
// bytes for splitting K over two workgroups per tile in a round that fills at
// most half of the GPU, or NULL (no split).  xf16 as for the GEMV.
size_t gemm_workspace_bytes(int64_t M, int64_t K, int64_t N, int G);
// The fixed device scratch of gq_w4a16_gemm_noalloc (GQ_NOALLOC_SCRATCH_BYTES,
// enough for the split of any 256-CU round): its address on the current
// device, looked up once per device; nullptr with *err set on failure.
constexpr size_t kNoAllocScratchBytes = GQ_NOALLOC_SCRATCH_BYTES;
void* noalloc_scratch(hipError_t* err);
hipError_t launch_w4a16_gemm(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                             const uint16_t* scales, const uint16_t* zeros, int64_t N, int G,
                             int symmetric, uint16_t* y, void* workspace, bool xf16, hipStream_t s);
hipError_t launch_q4k_quantize(const void* w, gq_dtype dt, int64_t N, int64_t K, uint8_t* blocks,
                               hipStream_t s);
// Super-block GEMV on the matrix cores (5 <= M <= 16, K a multiple of 512).
bool q4k_mfma_stream_supported(int M, int64_t K, int64_t N);
hipError_t launch_q4k_gemv_mfma_stream(const uint16_t* x, int M, int64_t K, const uint8_t* blocks,
                                       int64_t N, uint16_t* y, hipStream_t s);
hipError_t launch_q4k_gemv(const uint16_t* x, int M, int64_t K, const uint8_t* blocks, int64_t N,
                           uint16_t* y, hipStream_t s);

// Comparators and probes (no quantization): plain bf16 GEMV, 1 <= M <= 4, with
// x staged in M * bf16_gemv_kpad(K) * 2 bytes of LDS; HBM stream read.
int bf16_gemv_kpad(int64_t K);
hipError_t launch_bf16_gemv(const uint16_t* x, int M, int64_t K, const uint16_t* w, int64_t N,
                            uint16_t* y, hipStream_t s);
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_probe_mfma_valu(int valu, int iters, int grid, uint64_t* cycles, float* sink,
                                  hipStream_t s);
hipError_t launch_probe_lds_read(int waves, int iters, int grid, uint64_t* cycles, float* sink,
                                 hipStream_t s);

}  // namespace gq
