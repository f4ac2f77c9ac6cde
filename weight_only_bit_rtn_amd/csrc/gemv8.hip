// gemv8.hip -- the 8-bit instantiations of the dequant-GEMV kernel.
#include "gemv_kernel.h"

namespace lowbit {
template hipError_t launch_qgemv_bits<8>(const uint16_t*, int, const uint32_t*, const uint16_t*,
                                          const int32_t*, int, int, int, int, int, bool,
                                          uint16_t*, hipStream_t);
}  // namespace lowbit
