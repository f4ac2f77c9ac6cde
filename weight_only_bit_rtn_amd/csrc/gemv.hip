// gemv.hip -- dispatch of the dequant-GEMV by bit width and batch size.
//
// Batches 1..8 run on the VALU kernel (gemv_kernel.h), in passes of four
// rows when the activations of all rows do not fit the on-chip staging
// budget; grouped 2- and 4-bit codes take the small-batch matrix-core kernel
// (gemv_mma.hip) where it was measured faster.  Otherwise, from 9 rows on,
// and when even four rows do not fit, the product goes to the matrix-core
// GEMM (gemm.hip): at those batch sizes the per-weight work is dominated by
// the batch-many multiply-adds, which the fp16 MFMA units do for free while
// the VALU only decodes.
#include "common.h"
#include "kernels.h"

namespace lowbit {

template <int BITS>
hipError_t launch_qgemv_bits(const uint16_t* x, int B, const uint32_t* packed,
                             const uint16_t* scales, const int32_t* zeros, int N, int K, int G,
                             int gsz, int gshift, bool meta, uint16_t* y, hipStream_t stream);

constexpr int kGemvMaxValuBatch = 8;
constexpr int kGemvPassBatch = 4;  // rows per pass when all rows do not fit on chip

namespace {

hipError_t launch_rows(const uint16_t* x, int B, const uint32_t* packed, const uint16_t* scales,
                       const int32_t* zeros, int N, int K, int G, int gsz, int gshift, int bits,
                       bool meta, uint16_t* y, hipStream_t stream) {
  switch (bits) {
    case 2:
      return launch_qgemv_bits<2>(x, B, packed, scales, zeros, N, K, G, gsz, gshift, meta, y,
                                  stream);
    case 3:
      return launch_qgemv_bits<3>(x, B, packed, scales, zeros, N, K, G, gsz, gshift, meta, y,
                                  stream);
    case 8:
      return launch_qgemv_bits<8>(x, B, packed, scales, zeros, N, K, G, gsz, gshift, meta, y,
                                  stream);
    default:
      return launch_qgemv_bits<4>(x, B, packed, scales, zeros, N, K, G, gsz, gshift, meta, y,
                                  stream);
  }
}

}  // namespace

hipError_t launch_qgemv(const uint16_t* x, int64_t B, const uint32_t* packed,
                        const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K,
                        int bits, int64_t group_size, bool meta, uint16_t* y,
                        hipStream_t stream) {
  // Grouped 2- and 4-bit codes may take the small-batch matrix-core form
  // (gemv_mma.hip), which decodes each weight once for all activation rows
  // but pays a longer start-up and stages the activations in rounds whose
  // length shrinks with the tiles per workgroup.  Crossovers measured on
  // MI355X (Llama-7B 2-bit g64 MLP layers, 4-bit g128 layers of 2048 x 2048
  // and 28672 x 8192): on layers of at least one 16-row tile per CU it wins
  // from 5 rows on with up to three tiles per CU and from 4 rows on with one;
  // against the GEMM it wins from 9 rows on at any height up to three tiles
  // per CU; on layers of more than three tiles per CU the GEMM wins from 5
  // rows on.
  const bool grouped24 = group_size != 0 && (bits == 2 || bits == 4);
  const int cus = device_cu_count();
  const int64_t NT = (N + 15) / 16;
  const int64_t tiles_per_cu = (NT + cus - 1) / cus;
  const bool mma_suited = grouped24 && tiles_per_cu <= 3;
  const bool mma_first =
      mma_suited && (B > kGemvMaxValuBatch ||
                     (NT >= cus && (B > kGemvPassBatch || (B == kGemvPassBatch && tiles_per_cu == 1))));
  if (mma_first) {
    const hipError_t e = launch_qgemv_mma(x, B, packed, scales, zeros, N, K, bits, group_size,
                                          meta, y, stream);
    if (e != hipErrorNotSupported) return e;
  }
  if (grouped24 && !mma_suited && B > kGemvPassBatch) return hipErrorNotSupported;
  if (B > kGemvMaxValuBatch) return hipErrorNotSupported;
  const int gsz = (int)(group_size == 0 ? K : group_size);
  const int G = (int)(K / gsz);
  const int gshift = (gsz & (gsz - 1)) == 0 ? __builtin_ctz((unsigned)gsz) : -1;
  const int b = (int)B, n = (int)N, k = (int)K;
  hipError_t e = launch_rows(x, b, packed, scales, zeros, n, k, G, gsz, gshift, bits, meta, y,
                             stream);
  if (e != hipErrorNotSupported || b <= kGemvPassBatch) return e;
  if (mma_suited && NT >= cus) {
    e = launch_qgemv_mma(x, B, packed, scales, zeros, N, K, bits, group_size, meta, y, stream);
    if (e != hipErrorNotSupported) return e;
  }
  // The activations of all rows do not fit on chip: passes of up to four rows
  // (the weights are read once per pass, which costs less than the matrix-core
  // path at these batch sizes).  Every pass has the on-chip needs of the first
  // or fewer, so either the first is refused and nothing runs, or all run.
  for (int b0 = 0; b0 < b; b0 += kGemvPassBatch) {
    const int bc = b - b0 < kGemvPassBatch ? b - b0 : kGemvPassBatch;
    e = launch_rows(x + (int64_t)b0 * K, bc, packed, scales, zeros, n, k, G, gsz, gshift, bits,
                    meta, y + (int64_t)b0 * N, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lowbit
