// C ABI of libgq: argument validation, device check and dispatch to the
// kernels.  Validation runs entirely on the host before any HIP call, so an
// invalid call never touches the device (and can be exercised without one).
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstring>
#include <random>

#include "gq_internal.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other architecture
std::atomic<int> g_arch_state[kMaxDevices];
// compute-unit count per device (0 = unknown)
std::atomic<int> g_num_cus[kMaxDevices];

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

gq_status check_device(hipStream_t stream) {
  (void)stream;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GQ_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return GQ_ERR_UNSUPPORTED;
  int st = g_arch_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GQ_ERR_HIP;
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_num_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    g_arch_state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? GQ_OK : GQ_ERR_UNSUPPORTED;
}

gq_status from_hip(hipError_t e) { return e == hipSuccess ? GQ_OK : GQ_ERR_HIP; }

bool valid_dtype(gq_dtype d) { return d == GQ_F32 || d == GQ_F16 || d == GQ_BF16; }

constexpr int64_t kMaxDim = (int64_t)1 << 30;
// The GEMM addresses a 256-row activation tile with 32-bit byte offsets.
constexpr int64_t kMaxGemmK = (int64_t)1 << 22;

// Shape/group checks common to everything that reads or writes groups.
gq_status check_groups(int64_t N, int64_t K, int32_t G) {
  if (N < 0 || K < 1 || N > kMaxDim || K > kMaxDim) return GQ_ERR_INVALID_ARG;
  if (G < 32 || G % 32 != 0 || K % G != 0) return GQ_ERR_INVALID_ARG;
  if (N * (K / G) >= ((int64_t)1 << 31)) return GQ_ERR_INVALID_ARG;
  return GQ_OK;
}

// Checks shared by the packed 4-bit matmuls.
gq_status check_w4_matmul(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                          const uint16_t* scales, const uint16_t* zeros, int64_t N,
                          gq_qparams p, uint16_t* y) {
  if (M < 0 || M > kMaxDim) return GQ_ERR_INVALID_ARG;
  if (gq_status s = check_groups(N, K, p.group_size)) return s;
  if (p.symmetric != 0 && p.symmetric != 1) return GQ_ERR_INVALID_ARG;
  if (p.bits < 2 || p.bits > 8) return GQ_ERR_INVALID_ARG;
  if (p.bits != 4) return GQ_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return GQ_OK;
  if (!x || !qweight || !scales || !y) return GQ_ERR_INVALID_ARG;
  if ((zeros == nullptr) != (p.symmetric == 1)) return GQ_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(qweight) || !aligned16(y)) return GQ_ERR_MISALIGNED;
  return GQ_OK;
}

}  // namespace

namespace gq {

uint64_t next_launch_id() {
  static std::atomic<uint64_t> seq{[] {
    std::random_device rd;
    uint64_t v = ((uint64_t)rd() << 32) ^ (uint64_t)rd();
    v ^= (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() * 0x9E3779B97F4A7C15ull;
    return v;
  }()};
  return seq.fetch_add(2, std::memory_order_relaxed) | 1ull;
}

int num_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  const int n = g_num_cus[dev].load(std::memory_order_relaxed);
  return n > 0 ? n : 256;
}

}  // namespace gq

extern "C" {

const char* gq_status_str(gq_status s) {
  switch (s) {
    case GQ_OK: return "GQ_OK";
    case GQ_ERR_INVALID_ARG: return "GQ_ERR_INVALID_ARG: argument violates the contract";
    case GQ_ERR_UNSUPPORTED: return "GQ_ERR_UNSUPPORTED: not implemented for these parameters or this device";
    case GQ_ERR_MISALIGNED: return "GQ_ERR_MISALIGNED: pointer must be 16-byte aligned";
    case GQ_ERR_HIP: return "GQ_ERR_HIP: HIP runtime error";
  }
  return "unknown gq_status";
}

int32_t gq_version(void) { return 100; }

gq_status gq_packed_sizes(int64_t N, int64_t K, gq_qparams p, int64_t* qweight_bytes,
                          int64_t* scale_bytes, int64_t* zero_bytes) {
  if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim) return GQ_ERR_INVALID_ARG;
  if (p.bits < 2 || p.bits > 8) return GQ_ERR_INVALID_ARG;
  if (p.group_size < 1 || K % p.group_size != 0) return GQ_ERR_INVALID_ARG;
  if (p.symmetric != 0 && p.symmetric != 1) return GQ_ERR_INVALID_ARG;
  const int64_t groups = N * (K / p.group_size);
  if (qweight_bytes) *qweight_bytes = (N * K * p.bits + 7) / 8;
  if (scale_bytes) *scale_bytes = 2 * groups;
  if (zero_bytes) *zero_bytes = p.symmetric ? 0 : 2 * groups;
  return GQ_OK;
}

gq_status gq_quantize_groups(const void* w, gq_dtype w_dtype, int64_t N, int64_t K, gq_qparams p,
                             void* codes, uint16_t* scales, uint16_t* zeros, void* stream) {
  if (gq_status s = check_groups(N, K, p.group_size)) return s;
  if (p.bits < 2 || p.bits > 8) return GQ_ERR_INVALID_ARG;
  if (p.symmetric != 0 && p.symmetric != 1) return GQ_ERR_INVALID_ARG;
  if (!valid_dtype(w_dtype)) return GQ_ERR_INVALID_ARG;
  if (N == 0) return GQ_OK;
  if (!w || !codes || !scales) return GQ_ERR_INVALID_ARG;
  if ((zeros == nullptr) != (p.symmetric == 1)) return GQ_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (gq_status st = check_device(s)) return st;
  return from_hip(gq::launch_quantize_groups(w, w_dtype, N, K, p.bits, p.group_size, p.symmetric,
                                             codes, scales, zeros, s));
}

gq_status gq_pack_int4(const void* codes, int64_t N, int64_t K, int32_t symmetric,
                       uint8_t* qweight, void* stream) {
  if (N < 0 || K < 2 || N > kMaxDim || K > kMaxDim || (K & 1)) return GQ_ERR_INVALID_ARG;
  if (symmetric != 0 && symmetric != 1) return GQ_ERR_INVALID_ARG;
  if (N == 0) return GQ_OK;
  if (!codes || !qweight) return GQ_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (gq_status st = check_device(s)) return st;
  return from_hip(gq::launch_pack_int4(codes, N, K, symmetric, qweight, s));
}

gq_status gq_dequantize(const uint8_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                        int64_t N, int64_t K, gq_qparams p, void* w_hat, gq_dtype out_dtype,
                        void* stream) {
  if (gq_status s = check_groups(N, K, p.group_size)) return s;
  if (p.symmetric != 0 && p.symmetric != 1) return GQ_ERR_INVALID_ARG;
  if (p.bits < 2 || p.bits > 8) return GQ_ERR_INVALID_ARG;
  if (!valid_dtype(out_dtype)) return GQ_ERR_INVALID_ARG;
  if (p.bits != 4) return GQ_ERR_UNSUPPORTED;
  if (N == 0) return GQ_OK;
  if (!qweight || !scales || !w_hat) return GQ_ERR_INVALID_ARG;
  if ((zeros == nullptr) != (p.symmetric == 1)) return GQ_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (gq_status st = check_device(s)) return st;
  return from_hip(gq::launch_dequantize(qweight, scales, zeros, N, K, p.group_size, p.symmetric,
                                        w_hat, out_dtype, s));
}

gq_status gq_ingest_group_major(const int8_t* codes, const uint16_t* scales, int64_t n_groups,
                                int64_t group, int64_t N, uint8_t* qweight, uint16_t* scales_out,
                                void* stream) {
  if (n_groups < 1 || group < 1 || N < 0 || n_groups > kMaxDim || group > kMaxDim) return GQ_ERR_INVALID_ARG;
  if (gq_status st = check_groups(N, n_groups * group, (int32_t)group)) return st;
  if (N == 0) return GQ_OK;
  if (!codes || !scales || !qweight || !scales_out) return GQ_ERR_INVALID_ARG;
  if (!aligned16(qweight)) return GQ_ERR_MISALIGNED;
  hipStream_t s = (hipStream_t)stream;
  if (gq_status st = check_device(s)) return st;
  return from_hip(gq::launch_ingest_group_major(codes, scales, n_groups, group, N, qweight,
                                                scales_out, s));
}

}  // extern "C"

namespace {

// The GEMV entry points: validation, then the launch with the caller's
// workspace (or none) and the activation type.
gq_status gemv_call(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                    const uint16_t* scales, const uint16_t* zeros, int64_t N, gq_qparams p,
                    uint16_t* y, void* workspace, size_t workspace_bytes, bool has_ws, bool xf16,
                    void* stream) {
  if (M > 16) return GQ_ERR_INVALID_ARG;
  if (gq_status s = check_w4_matmul(x, M, K, qweight, scales, zeros, N, p, y)) return s;
  if (M == 0 || N == 0) return GQ_OK;
  const size_t need = has_ws ? gq::gemv_workspace_bytes((int)M, K, N, p.group_size) : 0;
  if (need > 0 && (!workspace || workspace_bytes < need)) return GQ_ERR_INVALID_ARG;
  if (need > 0 && !aligned16(workspace)) return GQ_ERR_MISALIGNED;
  hipStream_t s = (hipStream_t)stream;
  if (gq_status st = check_device(s)) return st;
  return from_hip(gq::launch_w4a16_gemv(x, (int)M, K, qweight, scales, zeros, N, p.group_size,
                                        p.symmetric, y, need ? workspace : nullptr, xf16, s));
}

// Limits of the GEMM launches: 32-bit tile counts and activation offsets.
gq_status check_gemm(int64_t M, int64_t K, int64_t N) {
  if (K > kMaxGemmK || M > kMaxDim / 2) return GQ_ERR_UNSUPPORTED;
  if (((M + 127) / 128) * ((N + 255) / 256) > INT32_MAX / 2) return GQ_ERR_UNSUPPORTED;
  return GQ_OK;
}

// The CU count the split decision uses: the device's when one is present.
void probe_device() {
  int n = 0;
  if (hipGetDeviceCount(&n) == hipSuccess && n > 0) (void)check_device(nullptr);
}

gq_status gemm_call(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                    const uint16_t* scales, const uint16_t* zeros, int64_t N, gq_qparams p,
                    uint16_t* y, void* workspace, size_t workspace_bytes, bool has_ws, bool xf16,
                    void* stream) {
  if (gq_status s = check_w4_matmul(x, M, K, qweight, scales, zeros, N, p, y)) return s;
  if (gq_status s = check_gemm(M, K, N)) return s;
  if (M == 0 || N == 0) return GQ_OK;
  size_t need = 0;
  if (has_ws) {
    probe_device();  // the split depends on the device's compute-unit count
    need = gq::gemm_workspace_bytes(M, K, N, p.group_size);
  }
  if (need > 0 && (!workspace || workspace_bytes < need)) return GQ_ERR_INVALID_ARG;
  if (need > 0 && !aligned16(workspace)) return GQ_ERR_MISALIGNED;
  hipStream_t s = (hipStream_t)stream;
  if (gq_status st = check_device(s)) return st;
  return from_hip(gq::launch_w4a16_gemm(x, M, K, qweight, scales, zeros, N, p.group_size,
                                        p.symmetric, y, need ? workspace : nullptr, xf16, s));
}

gq_status matmul_params(int64_t M, int64_t K, int64_t N, gq_qparams p) {
  if (M < 0 || M > kMaxDim) return GQ_ERR_INVALID_ARG;
  if (gq_status s = check_groups(N, K, p.group_size)) return s;
  if (p.symmetric != 0 && p.symmetric != 1) return GQ_ERR_INVALID_ARG;
  if (p.bits < 2 || p.bits > 8) return GQ_ERR_INVALID_ARG;
  if (p.bits != 4) return GQ_ERR_UNSUPPORTED;
  return GQ_OK;
}

}  // namespace

extern "C" {

gq_status gq_w4a16_gemv(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                        const uint16_t* scales, const uint16_t* zeros, int64_t N, gq_qparams p,
                        uint16_t* y, void* stream) {
  return gemv_call(x, M, K, qweight, scales, zeros, N, p, y, nullptr, 0, false, false, stream);
}

gq_status gq_w4a16_gemv_workspace_size(int64_t M, int64_t K, int64_t N, gq_qparams p,
                                       size_t* bytes) {
  if (!bytes) return GQ_ERR_INVALID_ARG;
  *bytes = 0;
  if (M > 16) return GQ_ERR_INVALID_ARG;
  if (gq_status s = matmul_params(M, K, N, p)) return s;
  *bytes = gq::gemv_workspace_bytes((int)M, K, N, p.group_size);
  return GQ_OK;
}

gq_status gq_w4a16_gemv_ws(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                           const uint16_t* scales, const uint16_t* zeros, int64_t N,
                           gq_qparams p, uint16_t* y, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return gemv_call(x, M, K, qweight, scales, zeros, N, p, y, workspace, workspace_bytes, true, false,
                   stream);
}

gq_status gq_w4a16_gemv_f16(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                            const uint16_t* scales, const uint16_t* zeros, int64_t N,
                            gq_qparams p, uint16_t* y, void* stream) {
  return gemv_call(x, M, K, qweight, scales, zeros, N, p, y, nullptr, 0, false, true, stream);
}

gq_status gq_w4a16_gemv_f16_ws(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                               const uint16_t* scales, const uint16_t* zeros, int64_t N,
                               gq_qparams p, uint16_t* y, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return gemv_call(x, M, K, qweight, scales, zeros, N, p, y, workspace, workspace_bytes, true, true,
                   stream);
}

gq_status gq_w4a16_gemm(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                        const uint16_t* scales, const uint16_t* zeros, int64_t N, gq_qparams p,
                        uint16_t* y, void* stream) {
  return gemm_call(x, M, K, qweight, scales, zeros, N, p, y, nullptr, 0, false, false, stream);
}

gq_status gq_w4a16_gemm_workspace_size(int64_t M, int64_t K, int64_t N, gq_qparams p,
                                       size_t* bytes) {
  if (!bytes) return GQ_ERR_INVALID_ARG;
  *bytes = 0;
  if (gq_status s = matmul_params(M, K, N, p)) return s;
  if (gq_status s = check_gemm(M, K, N)) return s;
  if (M == 0 || N == 0) return GQ_OK;
  probe_device();
  *bytes = gq::gemm_workspace_bytes(M, K, N, p.group_size);
  return GQ_OK;
}

gq_status gq_w4a16_gemm_ws(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                           const uint16_t* scales, const uint16_t* zeros, int64_t N,
                           gq_qparams p, uint16_t* y, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return gemm_call(x, M, K, qweight, scales, zeros, N, p, y, workspace, workspace_bytes, true, false,
                   stream);
}

gq_status gq_w4a16_gemm_noalloc(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                                const uint16_t* scales, const uint16_t* zeros, int64_t N,
                                gq_qparams p, uint16_t* y, void* stream) {
  if (gq_status s = check_w4_matmul(x, M, K, qweight, scales, zeros, N, p, y)) return s;
  if (gq_status s = check_gemm(M, K, N)) return s;
  if (M == 0 || N == 0) return GQ_OK;
  probe_device();  // the split depends on the device's compute-unit count
  const size_t need = gq::gemm_workspace_bytes(M, K, N, p.group_size);
  if (need > GQ_NOALLOC_SCRATCH_BYTES) return GQ_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  if (gq_status st = check_device(s)) return st;
  void* ws = nullptr;
  if (need > 0) {
    hipError_t e = hipSuccess;
    ws = gq::noalloc_scratch(&e);
    if (!ws) return GQ_ERR_HIP;
  }
  return from_hip(gq::launch_w4a16_gemm(x, M, K, qweight, scales, zeros, N, p.group_size,
                                        p.symmetric, y, ws, false, s));
}

gq_status gq_w4a16_gemm_f16(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                            const uint16_t* scales, const uint16_t* zeros, int64_t N,
                            gq_qparams p, uint16_t* y, void* stream) {
  return gemm_call(x, M, K, qweight, scales, zeros, N, p, y, nullptr, 0, false, true, stream);
}

gq_status gq_w4a16_gemm_f16_ws(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight,
                               const uint16_t* scales, const uint16_t* zeros, int64_t N,
                               gq_qparams p, uint16_t* y, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return gemm_call(x, M, K, qweight, scales, zeros, N, p, y, workspace, workspace_bytes, true, true,
                   stream);
}

gq_status gq_q4k_quantize(const void* w, gq_dtype w_dtype, int64_t N, int64_t K, uint8_t* blocks,
                          void* stream) {
  if (N < 0 || K < 256 || N > kMaxDim || K > kMaxDim || K % 256 != 0) return GQ_ERR_INVALID_ARG;
  if (!valid_dtype(w_dtype)) return GQ_ERR_INVALID_ARG;
  if (N == 0) return GQ_OK;
  if (!w || !blocks) return GQ_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (gq_status st = check_device(s)) return st;
  return from_hip(gq::launch_q4k_quantize(w, w_dtype, N, K, blocks, s));
}

gq_status gq_q4k_gemv(const uint16_t* x, int64_t M, int64_t K, const uint8_t* blocks, int64_t N,
                      uint16_t* y, void* stream) {
  if (M < 0 || M > 16) return GQ_ERR_INVALID_ARG;
  if (N < 0 || K < 256 || N > kMaxDim || K > kMaxDim || K % 256 != 0) return GQ_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return GQ_OK;
  if (!x || !blocks || !y) return GQ_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(blocks) || !aligned16(y)) return GQ_ERR_MISALIGNED;
  hipStream_t s = (hipStream_t)stream;
  if (gq_status st = check_device(s)) return st;
  return from_hip(gq::launch_q4k_gemv(x, (int)M, K, blocks, N, y, s));
}

gq_status gq_bf16_gemv(const uint16_t* x, int64_t M, int64_t K, const uint16_t* w, int64_t N,
                       uint16_t* y, void* stream) {
  if (M < 0 || M > 4) return GQ_ERR_INVALID_ARG;
  if (N < 0 || K < 8 || N > kMaxDim || K > kMaxDim || K % 8 != 0) return GQ_ERR_INVALID_ARG;
  if (N * K * 2 >= ((int64_t)1 << 31)) return GQ_ERR_UNSUPPORTED;
  if (M * (int64_t)gq::bf16_gemv_kpad(K) * 2 > 65536) return GQ_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return GQ_OK;
  if (!x || !w || !y) return GQ_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w) || ((uintptr_t)y & 1u)) return GQ_ERR_MISALIGNED;
  hipStream_t s = (hipStream_t)stream;
  if (gq_status st = check_device(s)) return st;
  return from_hip(gq::launch_bf16_gemv(x, (int)M, K, w, N, y, s));
}

gq_status gq_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (bytes < 0 || bytes % 16 != 0 || bytes > ((int64_t)1 << 38)) return GQ_ERR_INVALID_ARG;
  if (bytes == 0) return GQ_OK;
  if (!buf || !sink) return GQ_ERR_INVALID_ARG;
  if (!aligned16(buf) || ((uintptr_t)sink & 3u)) return GQ_ERR_MISALIGNED;
  hipStream_t s = (hipStream_t)stream;
  if (gq_status st = check_device(s)) return st;
  return from_hip(gq::launch_stream_read(buf, bytes, sink, s));
}

gq_status gq_probe_mfma_valu(int32_t valu, int32_t iters, int32_t grid, uint64_t* cycles, float* sink,
                             void* stream) {
  if (valu != 0 && valu != 32 && valu != 64 && valu != 128) return GQ_ERR_INVALID_ARG;
  if (iters < 1 || iters > (1 << 20) || grid < 1 || grid > 65536 || !cycles || !sink)
    return GQ_ERR_INVALID_ARG;
  if (((uintptr_t)cycles & 7u) || ((uintptr_t)sink & 3u)) return GQ_ERR_MISALIGNED;
  hipStream_t s = (hipStream_t)stream;
  if (gq_status st = check_device(s)) return st;
  return from_hip(gq::launch_probe_mfma_valu(valu, iters, grid, cycles, sink, s));
}

gq_status gq_probe_lds_read(int32_t waves, int32_t iters, int32_t grid, uint64_t* cycles, float* sink,
                            void* stream) {
  if (waves < 1 || waves > 16 || iters < 1 || iters > (1 << 20) || grid < 1 || grid > 65536 ||
      !cycles || !sink)
    return GQ_ERR_INVALID_ARG;
  if (((uintptr_t)cycles & 7u) || ((uintptr_t)sink & 3u)) return GQ_ERR_MISALIGNED;
  hipStream_t s = (hipStream_t)stream;
  if (gq_status st = check_device(s)) return st;
  return from_hip(gq::launch_probe_lds_read(waves, iters, grid, cycles, sink, s));
}

}  // extern "C"
