// gemv_kernel.h -- fused dequantize + matrix-vector product, batch 1..15, on the VALU.
//
// y[b][n] = sum_k x[b][k] * deq(packed[n])[k], with deq the exact fp16 value
// fp16_rne((q - z) * s) of min-max RTN.  The weights stay low-bit in HBM and
// are converted by the GPU's own cores inside the product ([Feature Request]
// 4bit and 2bit and 1bit quantization support: storing 4-bit weights on the
// GPU and converting them at run time); this is the weight-only mode that
// pays off when memory bandwidth is the constraint (BladeLLM model
// quantization, "Quantization modes", weight_only_quant).
//
// Work layout on gfx950:
//  - a workgroup is 4 waves; x (all B rows, all K) is staged once per
//    workgroup into LDS, already in the slot order the decode produces;
//  - each wave owns R consecutive weight rows at a time ("tile"); lane l owns
//    units l, l+64, ... of each row, so one load instruction of the wave
//    reads 1 KiB (2/4-bit) or 768 B (3-bit) of contiguous packed words;
//  - the wave walks a flat sequence of (tile, K step) iterations, loading the
//    next iteration's words (two register buffers) while decoding the
//    current one, so HBM reads stay in flight across tile boundaries;
//  - v_dot2_f32_f16 accumulates x * deq in fp32; at the end of a tile the 64
//    lanes are summed across the wave.
//  - one group per row: the row's constants are wave-uniform (scalar
//    registers); grouped rows take per-lane constants and "per-position"
//    accumulation (see unit_decode.h), which keeps the fast decode exact for
//    every normal scale.
#pragma once

#include "common.h"
#include "kernels.h"
#include "unit_decode.h"

namespace lowbit {

namespace gemv_detail {

constexpr int kGemvWaves = 4;
constexpr int kGemvThreads = kGemvWaves * kWave;
constexpr size_t kGemvLdsBudget = 64 * 1024;

// Unit a lane handles in K step j.
template <int BITS>
__device__ __forceinline__ UnitRef gemv_unit(int j, int lane, int K) {
  UnitRef u;
  if constexpr (BITS == 3) {
    const int pa = 128 * j + lane, pb = pa + 64;
    u.ka = 32 * pa;
    u.kb = 32 * pb;
    u.va = u.ka < K;
    u.vb = u.kb < K;
  } else {
    constexpr int C = Unit<BITS>::CODES;
    u.ka = C * (64 * j + lane);
    u.kb = u.ka;
    u.va = u.ka < K;
    u.vb = u.va;
  }
  return u;
}

template <int BITS>
constexpr int codes_per_step() {
  return 64 * Unit<BITS>::CODES;
}

// 2^-p of accumulator index i in per-position mode.
template <int BITS>
__device__ __forceinline__ float pos_scale(int i) {
  const int p = BITS == 4 ? 4 * i : BITS == 2 ? 2 * i : i;
  return 1.0f / (float)(1 << p);
}

__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

template <int BITS, int BB, int R, bool PERROW, bool SPLIT>
__global__ __launch_bounds__(kGemvThreads) void qgemv_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros,
    uint16_t* __restrict__ y, int N, int K, int G, int gsz, int gshift, int J, int Jfull) {
  using U = Unit<BITS>;
  constexpr int Q = U::QUADS, W = U::WORDS;
  constexpr bool POS = !PERROW;                      // per-position accumulation
  constexpr int NA = POS ? U::NPOS : 1;              // accumulators per (row, batch)
  constexpr int NC = (BITS == 2 && SPLIT) ? 2 : 1;   // constant sets per unit
  // scale/zero loads per row and unit: a 3-bit unit's two periods (lo / hi
  // halves) may sit in different groups, and so may a 2-bit unit's two periods
  constexpr int NL = (BITS == 3 && !PERROW) || (BITS == 2 && SPLIT) ? 2 : 1;
  extern __shared__ uint4 xs[];                      // [J][Q][BB][64], then slow scratch

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t wpr = (int64_t)K * BITS / 32;
  const int ntiles = (N + kGemvWaves * R - 1) / (kGemvWaves * R);
  const int mytiles = (int)blockIdx.x < ntiles ? (ntiles - 1 - (int)blockIdx.x) / (int)gridDim.x + 1
                                               : 0;
  const int total = mytiles * J;

  struct Buf {
    uint32_t w[R][W];
    uint16_t s[R][NL];
    int32_t z[R][NL];
  };

  auto row_of = [&](int it, int r) {
    const int k = it / J;
    const int tile = (int)blockIdx.x + k * (int)gridDim.x;
    const int n = (tile * kGemvWaves + wave) * R + r;
    return n < N ? n : N - 1;
  };

  auto load = [&](int it, Buf& b) {
    const int j = it % J;
    UnitRef u = gemv_unit<BITS>(j, lane, K);
    if (j >= Jfull) {  // past the end of the row: read unit 0 instead, masked later
      if (!u.va) u.ka = 0;
      if (!u.vb) u.kb = 0;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = row_of(it, r);
      const uint32_t* rowp = packed + (int64_t)n * wpr;
      if constexpr (BITS == 3) {
        const uint32_t* pa = rowp + 3 * (u.ka >> 5);
        const uint32_t* pb = rowp + 3 * (u.kb >> 5);
        b.w[r][0] = pa[0];
        b.w[r][1] = pa[1];
        b.w[r][2] = pa[2];
        b.w[r][3] = pb[0];
        b.w[r][4] = pb[1];
        b.w[r][5] = pb[2];
      } else {
        const uint4 v = *reinterpret_cast<const uint4*>(rowp + (u.ka * BITS >> 5));
        b.w[r][0] = v.x;
        b.w[r][1] = v.y;
        b.w[r][2] = v.z;
        b.w[r][3] = v.w;
      }
      if constexpr (PERROW) {
        if (j == 0) {
          b.s[r][0] = scales[n];
          b.z[r][0] = zeros[n];
        }
      } else {
        const uint16_t* srow = scales + (int64_t)n * G;
        const int32_t* zrow = zeros + (int64_t)n * G;
#pragma unroll
        for (int c = 0; c < NL; ++c) {
          const int kk = BITS == 3 ? (c == 0 ? u.ka : u.kb) : u.ka + 32 * c;
          const int g = group_of(kk, gsz, gshift);
          b.s[r][c] = srow[g];
          b.z[r][c] = zrow[g];
        }
      }
    }
  };

  // Prefetch the first iteration's weights before staging x, so the HBM
  // latency of the first loads overlaps the staging.
  Buf bufA, bufB;
  if (total > 0) load(0, bufA);

  const int entries = J * Q * BB * 64;
  uint32_t* slow_scratch = reinterpret_cast<uint32_t*>(xs + entries);
  for (int e = tid; e < entries; e += kGemvThreads) {
    const int l = e & 63;
    int rest = e >> 6;
    const int b = rest % BB;
    rest /= BB;
    const int q = rest % Q;
    const int j = rest / Q;
    const UnitRef u = gemv_unit<BITS>(j, l, K);
    xs[e] = x_entry<BITS>(x + (int64_t)b * K, u, q, true);
  }
  __syncthreads();

  float acc[R][BB][NA];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < BB; ++b)
#pragma unroll
      for (int a = 0; a < NA; ++a) acc[r][b][a] = 0.0f;

  const uint32_t mg = magic_register();
  Consts<BITS> rowc[R];
  uint16_t rows_s[R];
  int32_t rows_z[R];
  bool rowfast = true;

  auto compute = [&](int it, Buf& b) {
    const int j = it % J;
    const UnitRef u = gemv_unit<BITS>(j, lane, K);
    const bool tail = j >= Jfull;
    HalfParams hp[R][NC];
    Consts<BITS> cc[R][NC];
    bool fast = true;
    if constexpr (PERROW) {
      if (j == 0) {
        rowfast = true;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          rows_s[r] = (uint16_t)uniform(b.s[r][0]);
          rows_z[r] = (int32_t)uniform((uint32_t)b.z[r][0]);
          HalfParams h{rows_s[r], rows_s[r], rows_z[r], rows_z[r], true, true};
          rowfast &= make_consts<BITS, false>(h, rowc[r]);
#pragma unroll
          for (int i = 0; i < U::NPOS; ++i) {
            rowc[r].hz[i] = as_h2(uniform(as_u32(rowc[r].hz[i])));
            rowc[r].hs[i] = as_h2(uniform(as_u32(rowc[r].hs[i])));
          }
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        hp[r][0] = HalfParams{rows_s[r], rows_s[r], rows_z[r], rows_z[r], u.va, u.vb};
        cc[r][0] = rowc[r];
        if (tail) mask_consts<BITS, false>(cc[r][0], u.va, u.vb);
      }
      fast = rowfast;
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          if constexpr (BITS == 3)  // lo half from period a, hi half from period b
            hp[r][c] = HalfParams{b.s[r][0], b.s[r][1], b.z[r][0], b.z[r][1], u.va, u.vb};
          else
            hp[r][c] = HalfParams{b.s[r][c], b.s[r][c], b.z[r][c], b.z[r][c], u.va, u.vb};
          fast &= make_consts<BITS, true>(hp[r][c], cc[r][c]);
        }
      fast = __all(fast);
    }

    const uint4* xj = xs + (int64_t)j * Q * BB * 64 + lane;
    if (fast) {
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        uint4 xq[BB];
#pragma unroll
        for (int bb = 0; bb < BB; ++bb) xq[bb] = xj[(q * BB + bb) * 64];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int s = 4 * q + e;
            const int c = NC == 1 ? 0 : U::cset(s);
            const h2_t d = fast_pair<BITS, POS>(b.w[r], s, cc[r][c], mg);
            const int a = POS ? U::pidx(U::pos(s)) : 0;
#pragma unroll
            for (int bb = 0; bb < BB; ++bb) {
              const uint32_t xv = e == 0 ? xq[bb].x : e == 1 ? xq[bb].y : e == 2 ? xq[bb].z : xq[bb].w;
              acc[r][bb][a] = __builtin_amdgcn_fdot2(d, as_h2(xv), acc[r][bb][a], false);
            }
          }
      }
    } else {
      // Exact per-code path (rare: tiny or subnormal scales, zero points far
      // from the grid).  Kept compact: one slot per loop trip, the unit's
      // words read back from this wave's LDS scratch.
      uint32_t* wsc = slow_scratch + wave * (W * 64);
      const uint32_t* xj32 = reinterpret_cast<const uint32_t*>(xs + (int64_t)j * Q * BB * 64);
#pragma unroll
      for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int i = 0; i < W; ++i) wsc[i * 64 + lane] = b.w[r][i];
#pragma unroll 1
        for (int s = 0; s < U::SLOTS; ++s) {
          const int c = NC == 1 ? 0 : U::cset(s);
          const HalfParams h = c == 0 ? hp[r][0] : hp[r][NC - 1];
          const int ql = (int)unit_code_lds<BITS>(wsc, lane, U::lo(s));
          const int qh = (int)unit_code_lds<BITS>(wsc, lane, U::hi(s));
          const uint16_t dl = h.v_lo ? exact_deq(ql, h.z_lo, h_bits_to_f32(h.s_lo)) : (uint16_t)0;
          const uint16_t dh = h.v_hi ? exact_deq(qh, h.z_hi, h_bits_to_f32(h.s_hi)) : (uint16_t)0;
          const h2_t d = as_h2((uint32_t)dl | ((uint32_t)dh << 16));
          const int q = s >> 2, e = s & 3;
#pragma unroll
          for (int bb = 0; bb < BB; ++bb) {
            const uint32_t xv = xj32[((q * BB + bb) * 64 + lane) * 4 + e];
            acc[r][bb][0] = __builtin_amdgcn_fdot2(d, as_h2(xv), acc[r][bb][0], false);
          }
        }
      }
    }

    if (j == J - 1) {
      const int k = it / J;
      const int tile = (int)blockIdx.x + k * (int)gridDim.x;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int n = (tile * kGemvWaves + wave) * R + r;
#pragma unroll
        for (int bb = 0; bb < BB; ++bb) {
          float v = acc[r][bb][0];
#pragma unroll
          for (int a = 1; a < NA; ++a) v += acc[r][bb][a] * pos_scale<BITS>(a);
          v = wave_sum(v);
          if (lane == 0 && n < N) y[(int64_t)bb * N + n] = f32_to_h_bits(v);
#pragma unroll
          for (int a = 0; a < NA; ++a) acc[r][bb][a] = 0.0f;
        }
      }
    }
  };

  int it = 0;
  for (; it + 1 < total; it += 2) {
    load(it + 1, bufB);
    compute(it, bufA);
    if (it + 2 < total) load(it + 2, bufA);
    compute(it + 1, bufB);
  }
  if (it < total) compute(it, bufA);
}

template <int BITS, int BB, bool PERROW, bool SPLIT>
hipError_t launch_t(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                    const int32_t* zeros, int N, int K, int G, int gsz, int gshift, uint16_t* y,
                    hipStream_t stream) {
  constexpr int R = BB <= 4 ? 2 : 1;
  const int J = (K + codes_per_step<BITS>() - 1) / codes_per_step<BITS>();
  const int Jfull = K / codes_per_step<BITS>();
  const size_t lds = (size_t)J * Unit<BITS>::QUADS * BB * 64 * sizeof(uint4) +
                     (size_t)kGemvWaves * Unit<BITS>::WORDS * 64 * sizeof(uint32_t);
  if (lds > kGemvLdsBudget) return hipErrorNotSupported;
  const int ntiles = (N + kGemvWaves * R - 1) / (kGemvWaves * R);
  int per_cu = (int)(160 * 1024 / (lds + 1024));
  per_cu = per_cu < 1 ? 1 : per_cu > 4 ? 4 : per_cu;
  const int cap = device_cu_count() * per_cu;
  const int grid = ntiles < cap ? ntiles : cap;
  hipLaunchKernelGGL((qgemv_kernel<BITS, BB, R, PERROW, SPLIT>), dim3(grid), dim3(kGemvThreads),
                     lds, stream, x, packed, scales, zeros, y, N, K, G, gsz, gshift, J, Jfull);
  return hipGetLastError();
}

template <int BITS, bool PERROW, bool SPLIT>
hipError_t launch_bits(int B, const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                       const int32_t* zeros, int N, int K, int G, int gsz, int gshift,
                       uint16_t* y, hipStream_t stream) {
#define LOWBIT_GEMV_CASE(bb)                                                                  \
  case bb:                                                                                    \
    return launch_t<BITS, bb, PERROW, SPLIT>(x, packed, scales, zeros, N, K, G, gsz, gshift, \
                                             y, stream);
  switch (B) {
    LOWBIT_GEMV_CASE(1)
    LOWBIT_GEMV_CASE(2)
    LOWBIT_GEMV_CASE(3)
    LOWBIT_GEMV_CASE(4)
    LOWBIT_GEMV_CASE(5)
    LOWBIT_GEMV_CASE(6)
    LOWBIT_GEMV_CASE(7)
    LOWBIT_GEMV_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef LOWBIT_GEMV_CASE
}

}  // namespace gemv_detail

// Per-width entry (instantiated in gemv2.hip, gemv3.hip, gemv4.hip).
template <int BITS>
hipError_t launch_qgemv_bits(const uint16_t* x, int B, const uint32_t* packed,
                             const uint16_t* scales, const int32_t* zeros, int N, int K,
                             int G, int gsz, int gshift, uint16_t* y, hipStream_t stream) {
  using namespace gemv_detail;
  if (G == 1)
    return launch_bits<BITS, true, false>(B, x, packed, scales, zeros, N, K, G, gsz, gshift, y,
                                          stream);
  if constexpr (BITS == 2) {
    if (gsz % 64 != 0)
      return launch_bits<2, false, true>(B, x, packed, scales, zeros, N, K, G, gsz, gshift, y,
                                         stream);
  }
  return launch_bits<BITS, false, false>(B, x, packed, scales, zeros, N, K, G, gsz, gshift, y,
                                         stream);
}

}  // namespace lowbit
