// gemm.hip -- fused dequantize + small-batch matrix product on the fp16
// matrix cores (v_mfma_f32_16x16x32_f16 of gfx950).
//
// y[b][n] = sum_k x[b][k] * deq(packed[n])[k] with deq = fp16_rne((q - z) * s),
// the same contract as the matrix-vector kernel; this one is for batches
// where the product is a real dense contraction (16 and more activation rows).
// The weights are still decoded by the vector ALUs from their low-bit form
// ([Feature Request] 4bit and 2bit and 1bit quantization support: 4-bit
// weights kept on the GPU and converted by its cores at run time); the
// decoded fp16 values go straight from registers into the MFMA B operand.
//
// Tiling (one workgroup = 4 waves = 64 weight rows x 16*BT batch rows):
//  - MFMA 16x16x32: the 16 "columns" are 16 weight rows, the 16 "rows" are
//    16 batch rows, the 32-long contraction is 4 lane groups x 8 fp16 each;
//  - lane l of a wave decodes one unit (see unit_decode.h) of weight row
//    (l % 16); lane group h = l / 16 takes unit h of the current K tile, so a
//    K tile is 4 units (128 codes at 4 bits, 256 at 2 and 3 bits);
//  - a unit's slots 4s..4s+3 (8 fp16 values) are the B operand of MFMA step s;
//    the activation tile is staged in LDS in the same slot order (double
//    buffered), so the A operand is one 16-byte LDS read per lane and step;
//  - the contraction order inside the 32-long step is the slot order, which
//    is a permutation of k applied identically to both operands.
#include "common.h"
#include "kernels.h"
#include "unit_decode.h"

namespace lowbit {

namespace {

constexpr int kGemmWaves = 4;
constexpr int kGemmThreads = kGemmWaves * kWave;

template <int BITS>
__device__ __forceinline__ UnitRef gemm_unit(int t, int h, int K) {
  UnitRef u;
  if constexpr (BITS == 3) {
    const int pa = 8 * t + h, pb = pa + 4;
    u.ka = 32 * pa;
    u.kb = 32 * pb;
    u.va = u.ka < K;
    u.vb = u.kb < K;
  } else {
    constexpr int C = Unit<BITS>::CODES;
    u.ka = C * (4 * t + h);
    u.kb = u.ka;
    u.va = u.ka < K;
    u.vb = u.va;
  }
  return u;
}

template <int BITS>
constexpr int codes_per_tile() {
  return 4 * Unit<BITS>::CODES;
}

template <int BITS, int BT, bool PERROW>
__global__ __launch_bounds__(kGemmThreads) void qgemm_kernel(
    const uint16_t* __restrict__ x, int B, const uint32_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros,
    uint16_t* __restrict__ y, int N, int K, int G, int gsz, int gshift, int T) {
  using U = Unit<BITS>;
  constexpr int S = U::QUADS;  // MFMA steps per unit
  // [buffer][bt][s][h][i]: 16-byte A operands, lane (i, h) reads consecutive entries
  __shared__ uint4 xs[2][BT][S][4][16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, h = lane >> 4;
  const int n = blockIdx.x * (kGemmWaves * 16) + wave * 16 + i16;
  const bool nv = n < N;
  const int nn = nv ? n : N - 1;
  const int b0 = blockIdx.y * 16 * BT;
  const int64_t wpr = (int64_t)K * BITS / 32;
  const uint32_t* rowp = packed + (int64_t)nn * wpr;
  const uint16_t* srow = scales + (int64_t)nn * G;
  const int32_t* zrow = zeros + (int64_t)nn * G;

  auto stage = [&](int t, int buf) {
    // BT*S*4*16 entries, 256 threads
    for (int e = tid; e < BT * S * 64; e += kGemmThreads) {
      const int ei = e & 15, eh = (e >> 4) & 3;
      const int rest = e >> 6;
      const int es = rest % S, ebt = rest / S;
      const int b = b0 + 16 * ebt + ei;
      const UnitRef u = gemm_unit<BITS>(t, eh, K);
      const bool bv = b < B;
      xs[buf][ebt][es][eh][ei] = x_entry<BITS>(x + (int64_t)(bv ? b : 0) * K, u, es, bv);
    }
  };

  HalfParams rowp_;
  Consts<BITS> rowc[U::NCONST];
  bool rowfast = true;
  if constexpr (PERROW) {
    rowp_.s_lo = rowp_.s_hi = srow[0];
    rowp_.z_lo = rowp_.z_hi = zrow[0];
    rowp_.v_lo = rowp_.v_hi = true;
#pragma unroll
    for (int c = 0; c < U::NCONST; ++c) rowfast &= make_consts<BITS, false>(rowp_, rowc[c]);
  }

  const uint32_t mg = magic_register();
  f4_t acc[BT];
#pragma unroll
  for (int bt = 0; bt < BT; ++bt) acc[bt] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

  stage(0, 0);
  __syncthreads();
  for (int t = 0; t < T; ++t) {
    const int buf = t & 1;
    if (t + 1 < T) stage(t + 1, buf ^ 1);

    const UnitRef u = gemm_unit<BITS>(t, h, K);
    uint32_t w[U::WORDS];
    load_unit<BITS>(rowp, u, w);
    HalfParams hp[U::NCONST];
    Consts<BITS> cc[U::NCONST];
    bool fast = true;
    const bool full = u.va && u.vb;
    if constexpr (PERROW) {
#pragma unroll
      for (int c = 0; c < U::NCONST; ++c) {
        hp[c] = rowp_;
        if (full) {
          cc[c] = rowc[c];
        } else {
          hp[c].v_lo = u.va;
          hp[c].v_hi = u.vb;
          fast &= make_consts<BITS, false>(hp[c], cc[c]);
        }
      }
      if (full) fast = rowfast;
    } else {
#pragma unroll
      for (int c = 0; c < U::NCONST; ++c) {
        hp[c] = load_params<BITS>(srow, zrow, gsz, gshift, u, c);
        fast &= make_consts<BITS, false>(hp[c], cc[c]);
      }
    }

    h2_t bop[S][4];
    if (__all(fast)) {
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          bop[s][e] = fast_pair<BITS, false>(w, 4 * s + e, cc[U::cset(4 * s + e)], mg);
    } else {
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          bop[s][e] = slow_pair<BITS>(w, 4 * s + e, hp[U::cset(4 * s + e)]);
    }

#pragma unroll
    for (int s = 0; s < S; ++s) {
      const h8_t bv = __builtin_bit_cast(
          h8_t, make_uint4(as_u32(bop[s][0]), as_u32(bop[s][1]), as_u32(bop[s][2]),
                           as_u32(bop[s][3])));
#pragma unroll
      for (int bt = 0; bt < BT; ++bt) {
        const h8_t av = __builtin_bit_cast(h8_t, xs[buf][bt][s][h][i16]);
        acc[bt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc[bt], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // D layout: lane l holds rows 4*(l/16) + r (batch) of column l%16 (weight row)
  if (nv) {
#pragma unroll
    for (int bt = 0; bt < BT; ++bt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int b = b0 + 16 * bt + 4 * h + r;
        if (b < B) y[(int64_t)b * N + n] = f32_to_h_bits(acc[bt][r]);
      }
  }
}

template <int BITS, int BT, bool PERROW>
hipError_t launch_t(const uint16_t* x, int B, const uint32_t* packed, const uint16_t* scales,
                    const int32_t* zeros, int N, int K, int G, int gsz, int gshift, uint16_t* y,
                    hipStream_t stream) {
  const int T = (K + codes_per_tile<BITS>() - 1) / codes_per_tile<BITS>();
  const dim3 grid((unsigned)((N + kGemmWaves * 16 - 1) / (kGemmWaves * 16)),
                  (unsigned)((B + 16 * BT - 1) / (16 * BT)));
  hipLaunchKernelGGL((qgemm_kernel<BITS, BT, PERROW>), grid, dim3(kGemmThreads), 0, stream, x, B,
                     packed, scales, zeros, y, N, K, G, gsz, gshift, T);
  return hipGetLastError();
}

template <int BITS, bool PERROW>
hipError_t launch_bits(int B, const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                       const int32_t* zeros, int N, int K, int G, int gsz, int gshift,
                       uint16_t* y, hipStream_t stream) {
  if (B <= 16)
    return launch_t<BITS, 1, PERROW>(x, B, packed, scales, zeros, N, K, G, gsz, gshift, y, stream);
  if (B <= 32)
    return launch_t<BITS, 2, PERROW>(x, B, packed, scales, zeros, N, K, G, gsz, gshift, y, stream);
  return launch_t<BITS, 4, PERROW>(x, B, packed, scales, zeros, N, K, G, gsz, gshift, y, stream);
}

}  // namespace

hipError_t launch_qgemm(const uint16_t* x, int64_t B, const uint32_t* packed,
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
