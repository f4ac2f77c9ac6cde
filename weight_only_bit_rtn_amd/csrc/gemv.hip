// gemv.hip -- fused dequantize + matrix-vector product, batch 1..15, on the VALU.
//
// y[b][n] = sum_k x[b][k] * deq(packed[n])[k], with deq the exact fp16 value
// fp16_rne((q - z) * s) of min-max RTN.  The weights stay low-bit in HBM and
// are converted by the GPU's own cores inside the product ([Feature Request]
// 4bit and 2bit and 1bit quantization support: storing 4-bit weights on the
// GPU and converting them at run time); this is the weight-only mode that
// pays off when memory bandwidth is the constraint (BladeLLM model
// quantization, "Quantization modes", weight_only_quant).
//
// Layout of the work on gfx950:
//  - a workgroup is 4 waves; x (all B rows, all K) is staged once per
//    workgroup into LDS, already in the slot order the decode produces;
//  - each wave owns R consecutive weight rows at a time; lane l of the wave
//    owns units l, l+64, l+128, ... of every row, so one load instruction of
//    the wave reads 1 KiB (2-/4-bit) or 768 B (3-bit) of contiguous packed
//    words;
//  - the decode gives fp16 pairs; v_dot2_f32_f16 accumulates x * deq in
//    fp32;  at the end of the row the 64 lanes are summed across the wave.
//  - workgroups loop over row tiles (grid ~ a few workgroups per CU), so the
//    x staging is paid once per workgroup, not once per tile.
#include "common.h"
#include "kernels.h"
#include "unit_decode.h"

namespace lowbit {

namespace {

constexpr int kGemvWaves = 4;
constexpr int kGemvThreads = kGemvWaves * kWave;
constexpr size_t kGemvLdsBudget = 64 * 1024;

// Units a lane handles per iteration j, and the iteration count per row.
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
constexpr int codes_per_iter() {
  return 64 * Unit<BITS>::CODES;
}

template <int BITS, int BB, int R, bool PERROW>
__global__ __launch_bounds__(kGemvThreads) void qgemv_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros,
    uint16_t* __restrict__ y, int N, int K, int G, int gsz, int gshift, int J) {
  using U = Unit<BITS>;
  constexpr int Q = U::QUADS;
  extern __shared__ uint4 xs[];  // [J][Q][BB][64]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t wpr = (int64_t)K * BITS / 32;

  // Stage x into LDS in slot order (once per workgroup).
  const int entries = J * Q * BB * 64;
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

  const int ntiles = (N + kGemvWaves * R - 1) / (kGemvWaves * R);
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    int rows[R];
    bool rv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = (tile * kGemvWaves + wave) * R + r;
      rv[r] = n < N;
      rows[r] = rv[r] ? n : N - 1;
    }
    float acc[R][BB];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int b = 0; b < BB; ++b) acc[r][b] = 0.0f;

    // one group per row: the row's constants are loaded once
    HalfParams rowp[R];
    Consts<BITS> rowc[R][U::NCONST];
    bool rowfast = true;
    if constexpr (PERROW) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        rowp[r].s_lo = rowp[r].s_hi = scales[rows[r]];
        rowp[r].z_lo = rowp[r].z_hi = zeros[rows[r]];
        rowp[r].v_lo = rowp[r].v_hi = true;
#pragma unroll
        for (int c = 0; c < U::NCONST; ++c) rowfast &= make_consts<BITS>(rowp[r], rowc[r][c]);
      }
    }

    for (int j = 0; j < J; ++j) {
      const UnitRef u = gemv_unit<BITS>(j, lane, K);
      const bool full = u.va && u.vb;
      uint32_t w[R][U::WORDS];
#pragma unroll
      for (int r = 0; r < R; ++r) load_unit<BITS>(packed + rows[r] * wpr, u, w[r]);

      HalfParams hp[R][U::NCONST];
      Consts<BITS> cc[R][U::NCONST];
      bool fast = true;
      if constexpr (PERROW) {
        if (full) {
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < U::NCONST; ++c) {
              hp[r][c] = rowp[r];
              cc[r][c] = rowc[r][c];
            }
          fast = rowfast;
        } else {
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < U::NCONST; ++c) {
              hp[r][c] = rowp[r];
              hp[r][c].v_lo = u.va;
              hp[r][c].v_hi = u.vb;
              fast &= make_consts<BITS>(hp[r][c], cc[r][c]);
            }
        }
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int c = 0; c < U::NCONST; ++c) {
            hp[r][c] = load_params<BITS>(scales + (int64_t)rows[r] * G, zeros + (int64_t)rows[r] * G,
                                         gsz, gshift, u, c);
            fast &= make_consts<BITS>(hp[r][c], cc[r][c]);
          }
      }

      const uint4* xj = xs + (int64_t)j * Q * BB * 64 + lane;
      if (__all(fast)) {
#pragma unroll
        for (int q = 0; q < Q; ++q) {
          uint4 xq[BB];
#pragma unroll
          for (int b = 0; b < BB; ++b) xq[b] = xj[(q * BB + b) * 64];
#pragma unroll
          for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int s = 4 * q + e;
              const h2_t d = fast_pair<BITS>(w[r], s, cc[r][U::cset(s)]);
#pragma unroll
              for (int b = 0; b < BB; ++b) {
                const uint32_t xv = e == 0 ? xq[b].x : e == 1 ? xq[b].y : e == 2 ? xq[b].z : xq[b].w;
                acc[r][b] = __builtin_amdgcn_fdot2(d, as_h2(xv), acc[r][b], false);
              }
            }
          }
        }
      } else {
        for (int q = 0; q < Q; ++q) {
          uint4 xq[BB];
#pragma unroll
          for (int b = 0; b < BB; ++b) xq[b] = xj[(q * BB + b) * 64];
#pragma unroll
          for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int s = 4 * q + e;
              const h2_t d = slow_pair<BITS>(w[r], s, hp[r][U::cset(s)]);
#pragma unroll
              for (int b = 0; b < BB; ++b) {
                const uint32_t xv = e == 0 ? xq[b].x : e == 1 ? xq[b].y : e == 2 ? xq[b].z : xq[b].w;
                acc[r][b] = __builtin_amdgcn_fdot2(d, as_h2(xv), acc[r][b], false);
              }
            }
          }
        }
      }
    }

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int b = 0; b < BB; ++b) {
        const float v = wave_sum(acc[r][b]);
        if (lane == 0 && rv[r]) y[(int64_t)b * N + rows[r]] = f32_to_h_bits(v);
      }
  }
}

template <int BITS, int BB, bool PERROW>
hipError_t launch_t(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                    const int32_t* zeros, int N, int K, int G, int gsz, int gshift, uint16_t* y,
                    hipStream_t stream) {
  constexpr int R = BB <= 2 ? 4 : BB <= 8 ? 2 : 1;
  const int J = (K + codes_per_iter<BITS>() - 1) / codes_per_iter<BITS>();
  const size_t lds = (size_t)J * Unit<BITS>::QUADS * BB * 64 * sizeof(uint4);
  if (lds > kGemvLdsBudget) return hipErrorNotSupported;
  const int ntiles = (N + kGemvWaves * R - 1) / (kGemvWaves * R);
  int per_cu = (int)(160 * 1024 / (lds + 1024));
  per_cu = per_cu < 1 ? 1 : per_cu > 4 ? 4 : per_cu;
  const int cap = device_cu_count() * per_cu;
  const int grid = ntiles < cap ? ntiles : cap;
  hipLaunchKernelGGL((qgemv_kernel<BITS, BB, R, PERROW>), dim3(grid), dim3(kGemvThreads), lds,
                     stream, x, packed, scales, zeros, y, N, K, G, gsz, gshift, J);
  return hipGetLastError();
}

template <int BITS, bool PERROW>
hipError_t launch_bits(int B, const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                       const int32_t* zeros, int N, int K, int G, int gsz, int gshift,
                       uint16_t* y, hipStream_t stream) {
#define LOWBIT_GEMV_CASE(bb) \
  case bb:                   \
    return launch_t<BITS, bb, PERROW>(x, packed, scales, zeros, N, K, G, gsz, gshift, y, stream);
  switch (B) {
    LOWBIT_GEMV_CASE(1)
    LOWBIT_GEMV_CASE(2)
    LOWBIT_GEMV_CASE(3)
    LOWBIT_GEMV_CASE(4)
    LOWBIT_GEMV_CASE(5)
    LOWBIT_GEMV_CASE(6)
    LOWBIT_GEMV_CASE(7)
    LOWBIT_GEMV_CASE(8)
    LOWBIT_GEMV_CASE(9)
    LOWBIT_GEMV_CASE(10)
    LOWBIT_GEMV_CASE(11)
    LOWBIT_GEMV_CASE(12)
    LOWBIT_GEMV_CASE(13)
    LOWBIT_GEMV_CASE(14)
    LOWBIT_GEMV_CASE(15)
    default:
      return hipErrorInvalidValue;
  }
#undef LOWBIT_GEMV_CASE
}

}  // namespace

hipError_t launch_qgemv(const uint16_t* x, int64_t B, const uint32_t* packed,
                        const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K,
                        int bits, int64_t group_size, uint16_t* y, hipStream_t stream) {
  const int gsz = (int)(group_size == 0 ? K : group_size);
  const int G = (int)(K / gsz);
  const int gshift = (gsz & (gsz - 1)) == 0 ? __builtin_ctz((unsigned)gsz) : -1;
  const bool perrow = G == 1;
  const int b = (int)B, n = (int)N, k = (int)K;
  switch (bits) {
    case 2:
      return perrow ? launch_bits<2, true>(b, x, packed, scales, zeros, n, k, G, gsz, gshift, y, stream)
                    : launch_bits<2, false>(b, x, packed, scales, zeros, n, k, G, gsz, gshift, y, stream);
    case 3:
      return perrow ? launch_bits<3, true>(b, x, packed, scales, zeros, n, k, G, gsz, gshift, y, stream)
                    : launch_bits<3, false>(b, x, packed, scales, zeros, n, k, G, gsz, gshift, y, stream);
    default:
      return perrow ? launch_bits<4, true>(b, x, packed, scales, zeros, n, k, G, gsz, gshift, y, stream)
                    : launch_bits<4, false>(b, x, packed, scales, zeros, n, k, G, gsz, gshift, y, stream);
  }
}

}  // namespace lowbit
