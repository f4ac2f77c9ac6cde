// gemv.hip -- dispatch of the dequant-GEMV by bit width and batch size.
//
// Batches 1..8 run on the VALU kernel (gemv_kernel.h).  From 9 rows on, and
// whenever the activations do not fit the on-chip staging budget, the
// product goes to the matrix-core kernel (gemm.hip): at those batch sizes the
// per-weight work is dominated by the batch-many multiply-adds, which the
// fp16 MFMA units do for free while the VALU only decodes.
#include "kernels.h"

namespace lowbit {

template <int BITS>
hipError_t launch_qgemv_bits(const uint16_t* x, int B, const uint32_t* packed,
                             const uint16_t* scales, const int32_t* zeros, int N, int K, int G,
                             int gsz, int gshift, bool meta, uint16_t* y, hipStream_t stream);

constexpr int kGemvMaxValuBatch = 8;

hipError_t launch_qgemv(const uint16_t* x, int64_t B, const uint32_t* packed,
                        const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K,
                        int bits, int64_t group_size, bool meta, uint16_t* y,
                        hipStream_t stream) {
  if (B > kGemvMaxValuBatch) return hipErrorNotSupported;
  const int gsz = (int)(group_size == 0 ? K : group_size);
  const int G = (int)(K / gsz);
  const int gshift = (gsz & (gsz - 1)) == 0 ? __builtin_ctz((unsigned)gsz) : -1;
  const int b = (int)B, n = (int)N, k = (int)K;
  switch (bits) {
    case 2:
      return launch_qgemv_bits<2>(x, b, packed, scales, zeros, n, k, G, gsz, gshift, meta, y,
                                  stream);
    case 3:
      return launch_qgemv_bits<3>(x, b, packed, scales, zeros, n, k, G, gsz, gshift, meta, y,
                                  stream);
    case 8:
      return launch_qgemv_bits<8>(x, b, packed, scales, zeros, n, k, G, gsz, gshift, meta, y,
                                  stream);
    default:
      return launch_qgemv_bits<4>(x, b, packed, scales, zeros, n, k, G, gsz, gshift, meta, y,
                                  stream);
  }
}

}  // namespace lowbit
