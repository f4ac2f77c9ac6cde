// kernels.h -- internal host-side launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lowbit {

// Min-max grid (sym = false) or signed symmetric grid (sym = true).
hipError_t launch_quantize(const uint16_t* w, int64_t N, int64_t K, int bits, int64_t group_size,
                           bool sym, uint8_t* codes, uint32_t* packed, uint16_t* scales,
                           int32_t* zeros, hipStream_t stream);

hipError_t launch_pack(const uint8_t* codes, int64_t N, int64_t K, int bits, uint32_t* packed,
                       hipStream_t stream);

// Compact group words from separate scales and zeros (zero points saturated
// to int16, counted into *saturated when it is non-null).
hipError_t launch_pack_meta(const uint16_t* scales, const int32_t* zeros, int64_t count,
                            uint32_t* meta, int32_t* saturated, hipStream_t stream);

// Error-feedback (GPTQ) quantization in fp64; the workspace holds a status
// word, the K x K Hessian factor, the K x N residuals and N x K codes.
size_t gptq_workspace_bytes(int64_t N, int64_t K);
hipError_t launch_gptq(const uint16_t* w, int64_t N, int64_t K, const uint16_t* x,
                       int64_t n_samples, double damp, int bits, int64_t group_size, bool sym,
                       uint8_t* codes, uint32_t* packed, uint16_t* scales, int32_t* zeros,
                       void* workspace, hipStream_t stream);

// The same in the library's own static device scratch (kGptqScratchBytes per
// device; the caller checks gptq_workspace_bytes(N, K) against it): no
// allocation.  The run's status word is copied to *status_out when it is
// non-null.  Calls that overlap on one device race on the scratch.
constexpr size_t kGptqScratchBytes = (size_t)72 << 20;
hipError_t launch_gptq_noalloc(const uint16_t* w, int64_t N, int64_t K, const uint16_t* x,
                               int64_t n_samples, double damp, int bits, int64_t group_size,
                               uint8_t* codes, uint32_t* packed, uint16_t* scales, int32_t* zeros,
                               int32_t* status_out, hipStream_t stream);

// The products take the group parameters as separate scales and zeros, or
// (meta = true) as compact words passed through `scales` (zeros unused).

// Small-batch product on the matrix cores (1..16 activation rows) for 2- and
// 4-bit codes in groups of whole 16-byte units; hipErrorNotSupported for
// other layouts and for shares of work it is not sized for.
hipError_t launch_qgemv_mma(const uint16_t* x, int64_t B, const uint32_t* packed,
                            const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K,
                            int bits, int64_t group_size, bool meta, uint16_t* y,
                            hipStream_t stream);

// VALU dequant-GEMV; returns hipErrorNotSupported when x does not fit the
// on-chip staging budget (the caller then uses the MFMA path).
hipError_t launch_qgemv(const uint16_t* x, int64_t B, const uint32_t* packed,
                        const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K,
                        int bits, int64_t group_size, bool meta, uint16_t* y,
                        hipStream_t stream);

hipError_t launch_qgemm(const uint16_t* x, int64_t B, const uint32_t* packed,
                        const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K,
                        int bits, int64_t group_size, bool meta, uint16_t* y,
                        hipStream_t stream);

}  // namespace lowbit
