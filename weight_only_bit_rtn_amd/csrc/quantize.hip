// quantize.hip -- min-max round-to-nearest quantization and bitstream packing.
//
// Method: "MinMax" round-to-nearest with no calibration data (BladeLLM model
// quantization, "Quantization algorithms"), uniform asymmetric min-max grid
// per row (OPTQ reproducibility card, "Experiment Setup" row) or per block of
// consecutive input channels (BladeLLM "block_wise_quant").  Codes are packed
// several to a word ([Feature Request] 4bit and 2bit and 1bit quantization
// support, comments on two 4-bit codes per byte and sixteen 2-bit codes per
// int32); the bit order (least significant first, 3-bit codes straddling
// words) is this library's choice.
//
// Both kernels are HBM-streaming passes; one thread owns whole 32-code
// "periods" (64 bytes of fp16 weights, BITS words of packed codes), so every
// period packs into whole 32-bit words and every lane's loads and stores are
// contiguous with its neighbours'.
#include "common.h"
#include "kernels.h"

#pragma clang fp contract(off)

namespace lowbit {

namespace {

constexpr int kQuantThreads = 256;

template <int BITS>
__device__ __forceinline__ void pack_period(const uint32_t (&q)[32], uint32_t (&wd)[BITS]) {
#pragma unroll
  for (int i = 0; i < BITS; ++i) wd[i] = 0u;
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    const int bit = BITS * c;
    const int wi = bit >> 5;
    const int off = bit & 31;
    wd[wi] |= q[c] << off;
    if (off + BITS > 32) wd[wi + 1] |= q[c] >> (32 - off);
  }
}

template <int BITS>
__device__ __forceinline__ void store_packed(uint32_t* dst, const uint32_t (&wd)[BITS]) {
  if constexpr (BITS == 4) {
    *reinterpret_cast<uint4*>(dst) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  } else if constexpr (BITS == 2) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(wd[0], wd[1]);
  } else {
    dst[0] = wd[0];
    dst[1] = wd[1];
    dst[2] = wd[2];
  }
}

__device__ __forceinline__ void load_period_f32(const uint16_t* src, float (&v)[32]) {
  const uint4* p = reinterpret_cast<const uint4*>(src);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 u = p[i];
    const uint32_t d[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = h_bits_to_f32((uint16_t)(d[j] & 0xffffu));
      v[8 * i + 2 * j + 1] = h_bits_to_f32((uint16_t)(d[j] >> 16));
    }
  }
}

// One workgroup per row.  Three phases over the row:
//  1. per-period min/max into LDS,
//  2. per-group min/max -> (fp16 scale, int32 zero), written out and kept in LDS,
//  3. codes: q = clamp(rint(w / s) + z, 0, M), written as bytes and/or packed.
// Phase 3 re-reads the row, which the first phase has just brought into L2.
template <int BITS>
__global__ __launch_bounds__(kQuantThreads) void rtn_quantize_kernel(
    const uint16_t* __restrict__ w, int K, int gp /* periods per group */, int G,
    uint8_t* __restrict__ codes, uint32_t* __restrict__ packed, uint16_t* __restrict__ scales,
    int32_t* __restrict__ zeros) {
  constexpr int M = (1 << BITS) - 1;
  extern __shared__ float smem[];
  const int P = K >> 5;
  float* plo = smem;
  float* phi = smem + P;
  float* gsc = smem + 2 * P;
  int* gz = reinterpret_cast<int*>(smem + 2 * P + G);
  __shared__ float red_lo[kQuantThreads / kWave];
  __shared__ float red_hi[kQuantThreads / kWave];

  const int64_t row = blockIdx.x;
  const uint16_t* wr = w + row * (int64_t)K;
  const int tid = threadIdx.x;

  // phase 1
  for (int p = tid; p < P; p += kQuantThreads) {
    float v[32];
    load_period_f32(wr + 32 * p, v);
    float lo = v[0], hi = v[0];
#pragma unroll
    for (int c = 1; c < 32; ++c) {
      lo = fminf(lo, v[c]);
      hi = fmaxf(hi, v[c]);
    }
    plo[p] = lo;
    phi[p] = hi;
  }
  __syncthreads();

  // phase 2
  auto finish_group = [&](int j, float lo, float hi) {
    const float d = hi - lo;
    const float s32 = d / (float)M;
    uint16_t s16 = f32_to_h_bits(s32);
    if ((s16 & 0x7fffu) == 0) s16 = 0x3c00u;
    const float s = h_bits_to_f32(s16);
    const int z = (int)__builtin_rintf(-lo / s);
    scales[row * G + j] = s16;
    zeros[row * G + j] = z;
    gsc[j] = s;
    gz[j] = z;
  };
  if (gp <= 16) {
    for (int j = tid; j < G; j += kQuantThreads) {
      float lo = plo[j * gp], hi = phi[j * gp];
      for (int p = 1; p < gp; ++p) {
        lo = fminf(lo, plo[j * gp + p]);
        hi = fmaxf(hi, phi[j * gp + p]);
      }
      finish_group(j, lo, hi);
    }
  } else {
    const int wave = tid / kWave, lane = tid % kWave;
    for (int j = 0; j < G; ++j) {
      float lo = INFINITY, hi = -INFINITY;
      for (int p = tid; p < gp; p += kQuantThreads) {
        lo = fminf(lo, plo[j * gp + p]);
        hi = fmaxf(hi, phi[j * gp + p]);
      }
      lo = wave_min(lo);
      hi = wave_max(hi);
      if (lane == 0) {
        red_lo[wave] = lo;
        red_hi[wave] = hi;
      }
      __syncthreads();
      if (tid == 0) {
        for (int i = 1; i < kQuantThreads / kWave; ++i) {
          lo = fminf(lo, red_lo[i]);
          hi = fmaxf(hi, red_hi[i]);
        }
        finish_group(j, lo, hi);
      }
      __syncthreads();
    }
  }
  __syncthreads();

  // phase 3
  const int64_t wpr = (int64_t)K * BITS / 32;  // packed words per row
  for (int p = tid; p < P; p += kQuantThreads) {
    const int j = p / gp;
    const float s = gsc[j];
    const int z = gz[j];
    float v[32];
    load_period_f32(wr + 32 * p, v);
    uint32_t q[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      const int t = (int)__builtin_rintf(v[c] / s) + z;
      q[c] = (uint32_t)min(max(t, 0), M);
    }
    if (codes) {
      uint32_t b[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        b[i] = q[4 * i] | (q[4 * i + 1] << 8) | (q[4 * i + 2] << 16) | (q[4 * i + 3] << 24);
      uint4* dst = reinterpret_cast<uint4*>(codes + row * (int64_t)K + 32 * p);
      dst[0] = make_uint4(b[0], b[1], b[2], b[3]);
      dst[1] = make_uint4(b[4], b[5], b[6], b[7]);
    }
    if (packed) {
      uint32_t wd[BITS];
      pack_period<BITS>(q, wd);
      store_packed<BITS>(packed + row * wpr + (int64_t)BITS * p, wd);
    }
  }
}

// One thread per 32-code period of the whole [N][K] code matrix.
template <int BITS>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ codes, int64_t nper,
                                                   uint32_t* __restrict__ packed) {
  constexpr uint32_t mask = (1u << BITS) - 1u;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nper;
       i += (int64_t)gridDim.x * blockDim.x) {
    const uint4* src = reinterpret_cast<const uint4*>(codes + 32 * i);
    const uint4 a = src[0], b = src[1];
    const uint32_t by[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t q[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) q[c] = (by[c >> 2] >> (8 * (c & 3))) & mask;
    uint32_t wd[BITS];
    pack_period<BITS>(q, wd);
    store_packed<BITS>(packed + BITS * i, wd);
  }
}

}  // namespace

size_t quantize_lds_bytes(int64_t K, int64_t G) { return (size_t)(2 * (K / 32) + 2 * G) * 4; }

hipError_t launch_quantize(const uint16_t* w, int64_t N, int64_t K, int bits, int64_t gsz,
                           uint8_t* codes, uint32_t* packed, uint16_t* scales, int32_t* zeros,
                           hipStream_t stream) {
  const int64_t g = gsz == 0 ? K : gsz;
  const int64_t G = K / g;
  const int gp = (int)(g / 32);
  const size_t lds = quantize_lds_bytes(K, G);
  const dim3 grid((unsigned)N), block(kQuantThreads);
  switch (bits) {
    case 2:
      hipLaunchKernelGGL(rtn_quantize_kernel<2>, grid, block, lds, stream, w, (int)K, gp, (int)G,
                         codes, packed, scales, zeros);
      break;
    case 3:
      hipLaunchKernelGGL(rtn_quantize_kernel<3>, grid, block, lds, stream, w, (int)K, gp, (int)G,
                         codes, packed, scales, zeros);
      break;
    default:
      hipLaunchKernelGGL(rtn_quantize_kernel<4>, grid, block, lds, stream, w, (int)K, gp, (int)G,
                         codes, packed, scales, zeros);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_pack(const uint8_t* codes, int64_t N, int64_t K, int bits, uint32_t* packed,
                       hipStream_t stream) {
  const int64_t nper = N * (K / 32);
  const int64_t want = (nper + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 16;
  const dim3 grid((unsigned)(want < cap ? want : cap)), block(256);
  switch (bits) {
    case 2:
      hipLaunchKernelGGL(pack_kernel<2>, grid, block, 0, stream, codes, nper, packed);
      break;
    case 3:
      hipLaunchKernelGGL(pack_kernel<3>, grid, block, 0, stream, codes, nper, packed);
      break;
    default:
      hipLaunchKernelGGL(pack_kernel<4>, grid, block, 0, stream, codes, nper, packed);
      break;
  }
  return hipGetLastError();
}

}  // namespace lowbit
