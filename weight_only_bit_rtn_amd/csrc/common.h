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

// Round an fp64 value to the nearest fp16 (ties to even) directly from its
// bits: used where the exact value needs more than fp32's 24 bits, so a
// detour through fp32 would round twice.
__device__ inline uint16_t f64_to_h_bits(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const int e = (int)((b >> 52) & 0x7ff);
  uint64_t m = b & 0xFFFFFFFFFFFFFull;
  if (e == 0x7ff) return sign | 0x7c00u | (m ? 0x200u : 0u);
  if (e == 0) return sign;  // zero or an fp64 subnormal: far below fp16's range
  int E = e - 1023;
  m |= 1ull << 52;
  // bits of the 53-bit significand that fall below the fp16 quantum
  const int shift = (E >= -14) ? 42 : 42 + (-14 - E);
  if (shift > 54) return sign;
  uint64_t q = m >> shift;
  const uint64_t rem = m & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  if (E >= -14) {
    if (q == 2048) {
      q = 1024;
      ++E;
    }
    if (E > 15) return sign | 0x7c00u;
    return sign | (uint16_t)(((E + 15) << 10) | (int)(q - 1024));
  }
  return sign | (uint16_t)q;  // q == 1024 encodes the smallest normal
}

// Full-wave sum; every lane receives the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
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

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fminf(v, __shfl_xor(v, off, kWave));
  return v;
}

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
