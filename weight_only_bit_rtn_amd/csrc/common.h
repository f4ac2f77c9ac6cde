// common.h -- shared types and small device helpers of the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lowbit {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }
__device__ __forceinline__ uint32_t as_u32(h2_t v) { return __builtin_bit_cast(uint32_t, v); }

__device__ __forceinline__ float h_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}
// fp32 -> fp16, round to nearest even (v_cvt_f16_f32 in the default mode).
__device__ __forceinline__ uint16_t f32_to_h_bits(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)v);
}

// Sum over the 64 lanes with DPP lane permutations (no LDS traffic): pairs,
// quads, half rows, rows of 16, then the row broadcasts fold rows 0+1 into
// row 1, 2+3 into row 3 and finally everything into row 3.  Every lane gets
// the total (read from lane 63).
#define LOWBIT_DPP(v, ctrl, rmask)                                                     \
  __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), \
                                                        ctrl, rmask, 0xf, false))

__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += LOWBIT_DPP(v, 0xb1, 0xf);   // quad_perm [1,0,3,2]
  v += LOWBIT_DPP(v, 0x4e, 0xf);   // quad_perm [2,3,0,1]
  v += LOWBIT_DPP(v, 0x141, 0xf);  // row_half_mirror
  v += LOWBIT_DPP(v, 0x140, 0xf);  // row_mirror
  v += LOWBIT_DPP(v, 0x142, 0xa);  // row_bcast:15 into rows 1 and 3
  v += LOWBIT_DPP(v, 0x143, 0xc);  // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
#undef LOWBIT_DPP

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// Host side: compute-unit count of the current device, cached per device.
int device_cu_count();

// Host side: the largest LDS allocation one workgroup may make on the current
// device (bytes, cached per device).
size_t device_lds_per_block();

// Host side: allow `kernel` dynamic LDS allocations of up to `bytes` on the
// current device (hipFuncSetAttribute), once per kernel and device; safe to
// call from several host threads.
hipError_t raise_lds_limit(const void* kernel, int bytes);

}  // namespace lowbit
