// abi.hip -- the exported C entry points: argument checks, then launches.
//
// Every check runs on the host before anything is enqueued, so an error
// return means the stream was left untouched.
#include <stdint.h>

#include <mutex>
#include <set>
#include <utility>

#include "../../include/lowbit.h"
#include "common.h"
#include "kernels.h"

namespace lowbit {

int device_cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

size_t device_lds_per_block() {
  static std::mutex mu;
  static size_t cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 64 * 1024;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        v <= 0)
      v = 64 * 1024;
    cache[dev] = (size_t)v;
  }
  return cache[dev];
}

hipError_t raise_lds_limit(const void* kernel, int bytes) {
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;  // (kernel, device)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({kernel, dev})) return hipSuccess;
  const hipError_t e =
      hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.insert({kernel, dev});
  return e;
}

}  // namespace lowbit

static_assert(LOWBIT_GPTQ_NOALLOC_MAX_BYTES == lowbit::kGptqScratchBytes,
              "the header's scratch size and the library's must agree");

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_bits(int bits) {
  return (bits == 2 || bits == 3 || bits == 4 || bits == 8) ? LOWBIT_OK : LOWBIT_ERR_UNSUPPORTED;
}

int check_shape(int64_t N, int64_t K, int bits, int64_t group_size) {
  if (N < 0 || K < 0 || group_size < 0) return LOWBIT_ERR_ARG;
  if (N > INT32_MAX || K > INT32_MAX) return LOWBIT_ERR_SHAPE;
  if (K == 0 || K % 32 != 0 || (K * bits) % 128 != 0) return LOWBIT_ERR_SHAPE;
  if (group_size != 0 && (group_size % 32 != 0 || K % group_size != 0)) return LOWBIT_ERR_SHAPE;
  return LOWBIT_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? LOWBIT_OK : LOWBIT_ERR_HIP; }

// zeros == nullptr is accepted only with meta (compact words in `scales`).
int check_product(const void* x, int64_t B, const uint32_t* packed, const void* scales,
                  const int32_t* zeros, int64_t N, int64_t K, int bits, int64_t group_size,
                  const void* y, bool meta = false) {
  int rc = check_bits(bits);
  if (rc != LOWBIT_OK) return rc;
  if (B < 0) return LOWBIT_ERR_ARG;
  rc = check_shape(N, K, bits, group_size);
  if (rc != LOWBIT_OK) return rc;
  if (N == 0 || B == 0) return LOWBIT_OK;
  if (!x || !packed || !scales || (!meta && !zeros) || !y) return LOWBIT_ERR_ARG;
  if (!aligned16(x) || !aligned16(packed) || !aligned16(scales) ||
      (!meta && !aligned16(zeros)) || !aligned16(y))
    return LOWBIT_ERR_ARG;
  if ((int64_t)B * N > INT32_MAX || B > INT32_MAX) return LOWBIT_ERR_SHAPE;
  return LOWBIT_OK;
}

int quantize_checked(const void* w_f16, int64_t N, int64_t K, int bits, int64_t group_size,
                     bool sym, uint8_t* codes_or_null, uint32_t* packed_or_null,
                     uint16_t* scales_f16, int32_t* zeros, void* hip_stream) {
  int rc = check_bits(bits);
  if (rc != LOWBIT_OK) return rc;
  rc = check_shape(N, K, bits, group_size);
  if (rc != LOWBIT_OK) return rc;
  if (K > LOWBIT_QUANTIZE_MAX_K) return LOWBIT_ERR_SHAPE;
  if (N == 0) return LOWBIT_OK;
  if (!w_f16 || !scales_f16 || !zeros || (!codes_or_null && !packed_or_null))
    return LOWBIT_ERR_ARG;
  if (!aligned16(w_f16) || !aligned16(scales_f16) || !aligned16(zeros) ||
      (codes_or_null && !aligned16(codes_or_null)) ||
      (packed_or_null && !aligned16(packed_or_null)))
    return LOWBIT_ERR_ARG;
  return hip_status(lowbit::launch_quantize(static_cast<const uint16_t*>(w_f16), N, K, bits,
                                            group_size, sym, codes_or_null, packed_or_null,
                                            scales_f16, zeros,
                                            static_cast<hipStream_t>(hip_stream)));
}

}  // namespace

extern "C" {

int lowbit_quantize_rtn(const void* w_f16, int64_t N, int64_t K, int bits, int64_t group_size,
                        uint8_t* codes_or_null, uint32_t* packed_or_null, uint16_t* scales_f16,
                        int32_t* zeros, void* hip_stream) {
  return quantize_checked(w_f16, N, K, bits, group_size, false, codes_or_null, packed_or_null,
                          scales_f16, zeros, hip_stream);
}

int lowbit_quantize_rtn_sym(const void* w_f16, int64_t N, int64_t K, int bits,
                            int64_t group_size, uint8_t* codes_or_null, uint32_t* packed_or_null,
                            uint16_t* scales_f16, int32_t* zeros, void* hip_stream) {
  return quantize_checked(w_f16, N, K, bits, group_size, true, codes_or_null, packed_or_null,
                          scales_f16, zeros, hip_stream);
}

int lowbit_pack(const uint8_t* codes, int64_t N, int64_t K, int bits, uint32_t* packed,
                void* hip_stream) {
  int rc = check_bits(bits);
  if (rc != LOWBIT_OK) return rc;
  rc = check_shape(N, K, bits, 0);
  if (rc != LOWBIT_OK) return rc;
  if (N == 0) return LOWBIT_OK;
  if (!codes || !packed || !aligned16(codes) || !aligned16(packed)) return LOWBIT_ERR_ARG;
  return hip_status(
      lowbit::launch_pack(codes, N, K, bits, packed, static_cast<hipStream_t>(hip_stream)));
}

int lowbit_qgemv(const void* x_f16, int64_t B, const uint32_t* packed, const uint16_t* scales_f16,
                 const int32_t* zeros, int64_t N, int64_t K, int bits, int64_t group_size,
                 void* y_f16, void* hip_stream) {
  if (B > LOWBIT_QGEMV_MAX_B) return LOWBIT_ERR_ARG;
  int rc = check_product(x_f16, B, packed, scales_f16, zeros, N, K, bits, group_size, y_f16);
  if (rc != LOWBIT_OK || N == 0 || B == 0) return rc;
  const uint16_t* x = static_cast<const uint16_t*>(x_f16);
  uint16_t* y = static_cast<uint16_t*>(y_f16);
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  hipError_t e =
      lowbit::launch_qgemv(x, B, packed, scales_f16, zeros, N, K, bits, group_size, false, y, s);
  if (e == hipErrorNotSupported)  // x too large for on-chip staging: matrix-core path
    e = lowbit::launch_qgemm(x, B, packed, scales_f16, zeros, N, K, bits, group_size, false, y, s);
  return hip_status(e);
}

int lowbit_qgemm(const void* x_f16, int64_t B, const uint32_t* packed, const uint16_t* scales_f16,
                 const int32_t* zeros, int64_t N, int64_t K, int bits, int64_t group_size,
                 void* y_f16, void* hip_stream) {
  int rc = check_product(x_f16, B, packed, scales_f16, zeros, N, K, bits, group_size, y_f16);
  if (rc != LOWBIT_OK || N == 0 || B == 0) return rc;
  return hip_status(lowbit::launch_qgemm(static_cast<const uint16_t*>(x_f16), B, packed,
                                         scales_f16, zeros, N, K, bits, group_size, false,
                                         static_cast<uint16_t*>(y_f16),
                                         static_cast<hipStream_t>(hip_stream)));
}

int lowbit_pack_meta(const uint16_t* scales_f16, const int32_t* zeros, int64_t N, int64_t G,
                     uint32_t* meta, int32_t* saturated_or_null, void* hip_stream) {
  if (N < 0 || G < 0) return LOWBIT_ERR_ARG;
  if (N == 0 || G == 0) return LOWBIT_OK;
  if (N > INT64_MAX / G) return LOWBIT_ERR_SHAPE;
  if (!scales_f16 || !zeros || !meta) return LOWBIT_ERR_ARG;
  if (!aligned16(scales_f16) || !aligned16(zeros) || !aligned16(meta) ||
      (saturated_or_null && reinterpret_cast<uintptr_t>(saturated_or_null) % 4 != 0))
    return LOWBIT_ERR_ARG;
  return hip_status(lowbit::launch_pack_meta(scales_f16, zeros, N * G, meta, saturated_or_null,
                                             static_cast<hipStream_t>(hip_stream)));
}

int lowbit_qgemv_meta(const void* x_f16, int64_t B, const uint32_t* packed, const uint32_t* meta,
                      int64_t N, int64_t K, int bits, int64_t group_size, void* y_f16,
                      void* hip_stream) {
  if (B > LOWBIT_QGEMV_MAX_B) return LOWBIT_ERR_ARG;
  int rc = check_product(x_f16, B, packed, meta, nullptr, N, K, bits, group_size, y_f16, true);
  if (rc != LOWBIT_OK || N == 0 || B == 0) return rc;
  const uint16_t* x = static_cast<const uint16_t*>(x_f16);
  const uint16_t* m = reinterpret_cast<const uint16_t*>(meta);
  uint16_t* y = static_cast<uint16_t*>(y_f16);
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  hipError_t e = lowbit::launch_qgemv(x, B, packed, m, nullptr, N, K, bits, group_size, true, y, s);
  if (e == hipErrorNotSupported)  // x too large for on-chip staging: matrix-core path
    e = lowbit::launch_qgemm(x, B, packed, m, nullptr, N, K, bits, group_size, true, y, s);
  return hip_status(e);
}

int lowbit_qgemm_meta(const void* x_f16, int64_t B, const uint32_t* packed, const uint32_t* meta,
                      int64_t N, int64_t K, int bits, int64_t group_size, void* y_f16,
                      void* hip_stream) {
  int rc = check_product(x_f16, B, packed, meta, nullptr, N, K, bits, group_size, y_f16, true);
  if (rc != LOWBIT_OK || N == 0 || B == 0) return rc;
  return hip_status(lowbit::launch_qgemm(
      static_cast<const uint16_t*>(x_f16), B, packed, reinterpret_cast<const uint16_t*>(meta),
      nullptr, N, K, bits, group_size, true, static_cast<uint16_t*>(y_f16),
      static_cast<hipStream_t>(hip_stream)));
}

int64_t lowbit_gptq_workspace_bytes(int64_t N, int64_t K) {
  if (N < 0 || K <= 0 || K > LOWBIT_QUANTIZE_MAX_K || N > INT32_MAX) return LOWBIT_ERR_ARG;
  return (int64_t)lowbit::gptq_workspace_bytes(N, K);
}

static int gptq_checked(bool sym, const void* w_f16, int64_t N, int64_t K, const void* x_f16,
                        int64_t n_samples, double damp, int bits, int64_t group_size,
                        uint8_t* codes_or_null, uint32_t* packed_or_null, uint16_t* scales_f16,
                        int32_t* zeros, void* workspace, int64_t workspace_bytes,
                        void* hip_stream) {
  int rc = check_bits(bits);
  if (rc != LOWBIT_OK) return rc;
  rc = check_shape(N, K, bits, group_size);
  if (rc != LOWBIT_OK) return rc;
  if (K > LOWBIT_QUANTIZE_MAX_K || N > INT32_MAX) return LOWBIT_ERR_SHAPE;
  if (!(damp > 0.0) || !(damp < 1e300) || n_samples <= 0) return LOWBIT_ERR_ARG;
  if (N == 0) return LOWBIT_OK;
  if (!w_f16 || !x_f16 || !scales_f16 || !zeros || !workspace ||
      (!codes_or_null && !packed_or_null))
    return LOWBIT_ERR_ARG;
  if (!aligned16(w_f16) || !aligned16(x_f16) || !aligned16(scales_f16) || !aligned16(zeros) ||
      (codes_or_null && !aligned16(codes_or_null)) ||
      (packed_or_null && !aligned16(packed_or_null)) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return LOWBIT_ERR_ARG;
  if (workspace_bytes < (int64_t)lowbit::gptq_workspace_bytes(N, K)) return LOWBIT_ERR_ARG;
  return hip_status(lowbit::launch_gptq(
      static_cast<const uint16_t*>(w_f16), N, K, static_cast<const uint16_t*>(x_f16), n_samples,
      damp, bits, group_size, sym, codes_or_null, packed_or_null, scales_f16, zeros, workspace,
      static_cast<hipStream_t>(hip_stream)));
}

int lowbit_quantize_gptq(const void* w_f16, int64_t N, int64_t K, const void* x_f16,
                         int64_t n_samples, double damp, int bits, int64_t group_size,
                         uint8_t* codes_or_null, uint32_t* packed_or_null, uint16_t* scales_f16,
                         int32_t* zeros, void* workspace, int64_t workspace_bytes,
                         void* hip_stream) {
  return gptq_checked(false, w_f16, N, K, x_f16, n_samples, damp, bits, group_size,
                      codes_or_null, packed_or_null, scales_f16, zeros, workspace,
                      workspace_bytes, hip_stream);
}

int lowbit_quantize_gptq_sym(const void* w_f16, int64_t N, int64_t K, const void* x_f16,
                             int64_t n_samples, double damp, int bits, int64_t group_size,
                             uint8_t* codes_or_null, uint32_t* packed_or_null,
                             uint16_t* scales_f16, int32_t* zeros, void* workspace,
                             int64_t workspace_bytes, void* hip_stream) {
  return gptq_checked(true, w_f16, N, K, x_f16, n_samples, damp, bits, group_size,
                      codes_or_null, packed_or_null, scales_f16, zeros, workspace,
                      workspace_bytes, hip_stream);
}

int lowbit_quantize_gptq_noalloc(const void* w_f16, int64_t N, int64_t K, const void* x_f16,
                                 int64_t n_samples, double damp, int bits, int64_t group_size,
                                 uint8_t* codes_or_null, uint32_t* packed_or_null,
                                 uint16_t* scales_f16, int32_t* zeros, int32_t* status_or_null,
                                 void* hip_stream) {
  int rc = check_bits(bits);
  if (rc != LOWBIT_OK) return rc;
  rc = check_shape(N, K, bits, group_size);
  if (rc != LOWBIT_OK) return rc;
  if (K > LOWBIT_QUANTIZE_MAX_K || N > INT32_MAX) return LOWBIT_ERR_SHAPE;
  if (!(damp > 0.0) || !(damp < 1e300) || n_samples <= 0) return LOWBIT_ERR_ARG;
  if (N == 0) return LOWBIT_OK;
  if (!w_f16 || !x_f16 || !scales_f16 || !zeros || (!codes_or_null && !packed_or_null))
    return LOWBIT_ERR_ARG;
  if (!aligned16(w_f16) || !aligned16(x_f16) || !aligned16(scales_f16) || !aligned16(zeros) ||
      (codes_or_null && !aligned16(codes_or_null)) ||
      (packed_or_null && !aligned16(packed_or_null)) ||
      (status_or_null && (reinterpret_cast<uintptr_t>(status_or_null) & 3u) != 0))
    return LOWBIT_ERR_ARG;
  if (lowbit::gptq_workspace_bytes(N, K) > lowbit::kGptqScratchBytes) return LOWBIT_ERR_SCRATCH;
  return hip_status(lowbit::launch_gptq_noalloc(
      static_cast<const uint16_t*>(w_f16), N, K, static_cast<const uint16_t*>(x_f16), n_samples,
      damp, bits, group_size, codes_or_null, packed_or_null, scales_f16, zeros, status_or_null,
      static_cast<hipStream_t>(hip_stream)));
}

const char* lowbit_status_string(int status) {
  switch (status) {
    case LOWBIT_OK:
      return "ok";
    case LOWBIT_ERR_ARG:
      return "invalid argument (null or misaligned pointer, negative size, batch out of range)";
    case LOWBIT_ERR_SHAPE:
      return "unsupported shape (K must be a positive multiple of 32 with K*bits a multiple of "
             "128; group_size 0 or a multiple of 32 dividing K)";
    case LOWBIT_ERR_UNSUPPORTED:
      return "unsupported bit width (2, 3, 4 or 8)";
    case LOWBIT_ERR_HIP:
      return "HIP runtime error while launching";
    case LOWBIT_ERR_SCRATCH:
      return "problem larger than the static scratch of lowbit_quantize_gptq_noalloc "
             "(LOWBIT_GPTQ_NOALLOC_MAX_BYTES of workspace)";
    default:
      return "unknown status";
  }
}

}  // extern "C"
