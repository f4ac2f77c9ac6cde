// gemv_kernel.h -- fused dequantize + matrix-vector product, small batches, on the VALU.
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
//  - a workgroup is WAVES waves; x (all B rows, all K) is staged once per
//    workgroup into LDS, already in the slot order the decode produces;
//  - each wave owns R consecutive weight rows at a time ("tile"); lane l owns
//    units l, l+64, ... of each row, so one load instruction of the wave
//    reads 1 KiB (2/4-bit) or 768 B (3-bit) of contiguous packed words;
//  - loads are buffer loads with the streaming (slc) cache policy, which
//    measurably raises the HBM read rate on MI355X for data read once,
//    through a per-row resource descriptor whose size
//    is the row's byte count: lanes past the end of the row read zeros
//    instead of touching the next row (the range check applies to the vector
//    offset, so the K step is added there);
//  - the wave walks a flat sequence of (tile, K step) iterations, loading the
//    next iteration's words (two register buffers) while decoding the
//    current one, so HBM reads stay in flight across tile boundaries;
//  - v_dot2_f32_f16 accumulates x * deq in fp32; at the end of a tile the 64
//    lanes are summed with DPP permutations;
//  - one group per row: the row's constants are wave-uniform (scalar
//    registers); grouped rows take per-lane constants and per-position
//    accumulation (see unit_decode.h), which keeps the fast decode exact for
//    every normal scale.
#pragma once

#include "common.h"
#include "kernels.h"
#include "unit_decode.h"

namespace lowbit {

namespace gemv_detail {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr size_t kLdsBudget = 64 * 1024;
constexpr int kBufferDword3 = 0x00020000;  // raw 32-bit buffer format (gfx9 family)
constexpr int kSlc = 2;  // buffer-load cache policy for the weights: streaming

typedef uint32_t u3_t __attribute__((ext_vector_type(3)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferDword3);
}

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

// Bytes of packed words one K step covers (64 lanes).
template <int BITS>
constexpr int bytes_per_step() {
  return codes_per_step<BITS>() * BITS / 8;
}

// 2^-p of accumulator index i in per-position mode.
template <int BITS>
__device__ __forceinline__ float pos_scale(int i) {
  const int p = BITS == 4 ? 4 * i : BITS == 2 ? 2 * i : i;
  return 1.0f / (float)(1 << p);
}

// Order in which the matrix-vector kernel groups a unit's slots into quads
// (four fp16 pairs = one 16-byte activation entry = one MFMA operand).
// Scaled mode keeps the natural order; per-position mode puts slots of equal
// bit position together, so that every quad feeds a single accumulator.
template <int BITS, bool POS>
__host__ __device__ constexpr int quad_slot(int t, int e) {
  if constexpr (POS && BITS == 4) {
    constexpr int tab[16] = {0, 2, 4, 6, 8, 10, 12, 14, 1, 3, 5, 7, 9, 11, 13, 15};
    return tab[4 * t + e];
  } else if constexpr (POS && BITS == 2) {
    constexpr int tab[32] = {0, 5, 8, 13, 16, 21, 24, 29, 1, 6, 9, 14, 17, 22, 25, 30,
                             2, 7, 10, 15, 18, 23, 26, 31, 3, 11, 19, 27, 4, 12, 20, 28};
    return tab[4 * t + e];
  } else {
    return 4 * t + e;
  }
}

// Quad and element holding slot s (inverse of quad_slot).
template <int BITS, bool POS>
__host__ __device__ constexpr int slot_quad_elem(int s) {
  for (int t = 0; t < Unit<BITS>::QUADS; ++t)
    for (int e = 0; e < 4; ++e)
      if (quad_slot<BITS, POS>(t, e) == s) return 4 * t + e;
  return -1;
}

template <int BITS, bool POS>
constexpr bool quads_single_position() {
  using U = Unit<BITS>;
  bool seen[U::SLOTS] = {};
  for (int t = 0; t < U::QUADS; ++t)
    for (int e = 0; e < 4; ++e) {
      const int s = quad_slot<BITS, POS>(t, e);
      if (s < 0 || s >= U::SLOTS || seen[s]) return false;
      seen[s] = true;
      if (POS && U::pos(s) != U::pos(quad_slot<BITS, POS>(t, 0))) return false;
    }
  return true;
}
static_assert(quads_single_position<4, false>() && quads_single_position<4, true>() &&
                  quads_single_position<2, false>() && quads_single_position<2, true>() &&
                  quads_single_position<3, false>(),
              "quad orders must be permutations of the slots, one bit position per quad");

// Activation entry of quad t with slots in any order: eight 2-byte gathers.
template <int BITS, bool POS>
__device__ __forceinline__ uint4 x_entry_ordered(const uint16_t* __restrict__ xrow,
                                                 const UnitRef& u, int t) {
  using U = Unit<BITS>;
  if constexpr (!POS) {
    return x_entry<BITS>(xrow, u, t, true);
  } else {
    uint32_t d[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int s = quad_slot<BITS, POS>(t, e);
      const int cl = U::lo(s), ch = U::hi(s);
      const bool vl = BITS == 3 ? (cl < 32 ? u.va : u.vb) : u.va;
      const bool vh = BITS == 3 ? (ch < 32 ? u.va : u.vb) : u.va;
      const uint32_t a = vl ? xrow[unit_k<BITS>(u, cl)] : 0u;
      const uint32_t b = vh ? xrow[unit_k<BITS>(u, ch)] : 0u;
      d[e] = a | (b << 16);
    }
    return make_uint4(d[0], d[1], d[2], d[3]);
  }
}

// The diagonal element D[j][j] of a 16x16 MFMA accumulator that lane l
// holds: lanes whose column (l % 16) falls in their row block 4*(l / 16)
// .. +3 hold one diagonal element each (element l % 4); the others give 0.
__device__ __forceinline__ float mfma_diag(const f4_t& d, int lane) {
  const int e = lane & 3;
  const float v = e == 0 ? d[0] : e == 1 ? d[1] : e == 2 ? d[2] : d[3];
  return ((lane & 15) >> 2) == (lane >> 4) ? v : 0.0f;
}

__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

template <int BITS, int BB, int R, bool PERROW, bool SPLIT>
__global__ __launch_bounds__(kThreads) void qgemv_kernel(
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
  // Batch 1, one group per row: the multiply-accumulate runs on the matrix
  // cores (grouped layouts keep v_dot2: their per-position accumulators would
  // need one MFMA accumulator tile per bit position, which costs more
  // registers than it saves).  Each lane
  // puts its own 8 activations (A operand) and its own 8 dequantized weights
  // (B operand) into v_mfma_f32_16x16x32_f16; the diagonal D[j][j] of the
  // result is then the dot product over lanes j, j+16, j+32, j+48, and the
  // VALU only decodes.  (Off-diagonal entries mix lanes and are ignored.)
  constexpr bool MD = BB == 1 && PERROW;
  extern __shared__ uint4 xs[];                      // [J][Q][BB][64], then slow scratch

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t row_bytes = (uint32_t)K * BITS / 8;
  const int ntiles = (N + kWaves * R - 1) / (kWaves * R);
  const int mytiles = (int)blockIdx.x < ntiles ? (ntiles - 1 - (int)blockIdx.x) / (int)gridDim.x + 1
                                               : 0;
  const int total = mytiles * J;
  // per-lane byte offsets of the lane's unit inside one K step
  const uint32_t off_a = BITS == 3 ? 12u * lane : 16u * lane;
  const uint32_t off_b = off_a + 768u;

  struct Buf {
    uint32_t w[R][W];
    uint16_t s[R][NL];
    int32_t z[R][NL];
  };

  auto first_row = [&](int k) { return (((int)blockIdx.x + k * (int)gridDim.x) * kWaves + wave) * R; };

  const auto srs = rsrc(scales, (uint32_t)min((int64_t)N * G * 2, (int64_t)0x7fffffff));
  const auto zrs = rsrc(zeros, (uint32_t)min((int64_t)N * G * 4, (int64_t)0x7fffffff));
  auto load = [&](int k, int j, Buf& b) {
    const int n0 = first_row(k);
    const uint32_t step = (uint32_t)j * bytes_per_step<BITS>();
    const uint32_t va_off = off_a + step, vb_off = off_b + step;
    UnitRef u;
    if constexpr (!PERROW) u = gemv_unit<BITS>(j, lane, K);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = min(n0 + r, N - 1);
      const auto rs = rsrc(packed + (int64_t)n * (row_bytes / 4), row_bytes);
      if constexpr (BITS == 3) {
        const u3_t va = __builtin_amdgcn_raw_buffer_load_b96(rs, va_off, 0, kSlc);
        const u3_t vb = __builtin_amdgcn_raw_buffer_load_b96(rs, vb_off, 0, kSlc);
        b.w[r][0] = va.x;
        b.w[r][1] = va.y;
        b.w[r][2] = va.z;
        b.w[r][3] = vb.x;
        b.w[r][4] = vb.y;
        b.w[r][5] = vb.z;
      } else {
        const u4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, va_off, 0, kSlc);
        b.w[r][0] = v.x;
        b.w[r][1] = v.y;
        b.w[r][2] = v.z;
        b.w[r][3] = v.w;
      }
      if constexpr (PERROW) {
        if (j == 0) {
          // vector (buffer) loads on purpose: a scalar load would share the
          // lgkm counter with the LDS activation reads, and every wait on
          // those would then also wait for this prefetch to come from HBM
          const uint32_t nn = (uint32_t)n + 0u * (uint32_t)lane;
          b.s[r][0] = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(srs, 2u * nn, 0, 0);
          b.z[r][0] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(zrs, 4u * nn, 0, 0);
        }
      } else {
        const uint16_t* srow = scales + (int64_t)n * G;
        const int32_t* zrow = zeros + (int64_t)n * G;
#pragma unroll
        for (int c = 0; c < NL; ++c) {
          const int kk = BITS == 3 ? (c == 0 ? u.ka : u.kb) : u.ka + 32 * c;
          const bool v = BITS == 3 ? (c == 0 ? u.va : u.vb) : u.va;
          const int g = v ? group_of(kk, gsz, gshift) : 0;
          b.s[r][c] = srow[g];
          b.z[r][c] = zrow[g];
        }
      }
    }
  };

  // Prefetch the first iteration's weights before staging x, so the HBM
  // latency of the first loads overlaps the staging.
  Buf bufA, bufB;
  if (total > 0) load(0, 0, bufA);

  const int entries = J * Q * BB * 64;
  uint32_t* slow_scratch = reinterpret_cast<uint32_t*>(xs + entries);
  for (int e = tid; e < entries; e += kThreads) {
    const int l = e & 63;
    int rest = e >> 6;
    const int b = rest % BB;
    rest /= BB;
    const int q = rest % Q;
    const int j = rest / Q;
    const UnitRef u = gemv_unit<BITS>(j, l, K);
    xs[e] = MD ? x_entry_ordered<BITS, POS>(x + (int64_t)b * K, u, q)
               : x_entry<BITS>(x + (int64_t)b * K, u, q, true);
  }
  __syncthreads();

  float acc[R][BB][NA];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < BB; ++b)
#pragma unroll
      for (int a = 0; a < NA; ++a) acc[r][b][a] = 0.0f;
  f4_t dacc[R][MD ? NA : 1];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int a = 0; a < (MD ? NA : 1); ++a) dacc[r][a] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const uint32_t mg = magic_register();
  Consts<BITS> rowc[R];
  uint16_t rows_s[R];
  int32_t rows_z[R];
  bool rowfast = true;

  auto compute = [&](int k, int j, Buf& b) {
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
    if (MD && fast) {
#pragma unroll
      for (int t = 0; t < Q; ++t) {
        const h8_t av = __builtin_bit_cast(h8_t, xj[t * 64]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          h2_t d[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int s = quad_slot<BITS, POS>(t, e);
            const int c = NC == 1 ? 0 : U::cset(s);
            d[e] = fast_pair<BITS, POS>(b.w[r], s, cc[r][c], mg);
          }
          const h8_t bv = __builtin_bit_cast(
              h8_t, make_uint4(as_u32(d[0]), as_u32(d[1]), as_u32(d[2]), as_u32(d[3])));
          const int a = POS ? U::pidx(U::pos(quad_slot<BITS, POS>(t, 0))) : 0;
          dacc[r][MD ? a : 0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, dacc[r][MD ? a : 0], 0, 0, 0);
        }
      }
    } else if (!MD && fast) {
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
          const int qe = MD ? slot_quad_elem<BITS, POS>(s) : s;
          const int q = qe >> 2, e = qe & 3;
#pragma unroll
          for (int bb = 0; bb < BB; ++bb) {
            const uint32_t xv = xj32[((q * BB + bb) * 64 + lane) * 4 + e];
            acc[r][bb][0] = __builtin_amdgcn_fdot2(d, as_h2(xv), acc[r][bb][0], false);
          }
        }
      }
    }

    if (j == J - 1) {
      const int n0 = first_row(k);
#pragma unroll
      for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int bb = 0; bb < BB; ++bb) {
          float v = acc[r][bb][0];
#pragma unroll
          for (int a = 1; a < NA; ++a) v += acc[r][bb][a] * pos_scale<BITS>(a);
          if constexpr (MD) {
#pragma unroll
            for (int a = 0; a < NA; ++a) {
              v += mfma_diag(dacc[r][a], lane) * pos_scale<BITS>(a);
              dacc[r][a] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
            }
          }
          v = wave_sum_dpp(v);
          if (lane == 0 && n0 + r < N) y[(int64_t)bb * N + n0 + r] = f32_to_h_bits(v);
#pragma unroll
          for (int a = 0; a < NA; ++a) acc[r][bb][a] = 0.0f;
        }
      }
    }
  };

  // Two-deep software pipeline over the flat (tile k, K step j) sequence:
  // the loads of iteration i+1 are issued before iteration i is decoded.
  int ck = 0, cj = 0;  // iteration being computed
  int lk = 0, lj = 0;  // iteration most recently loaded
  auto advance = [&](int& k, int& j) {
    if (++j == J) {
      j = 0;
      ++k;
    }
  };
  int it = 0;
  for (; it + 1 < total; it += 2) {
    advance(lk, lj);
    load(lk, lj, bufB);
    compute(ck, cj, bufA);
    advance(ck, cj);
    if (it + 2 < total) {
      advance(lk, lj);
      load(lk, lj, bufA);
    }
    compute(ck, cj, bufB);
    advance(ck, cj);
  }
  if (it < total) compute(ck, cj, bufA);
}

template <int BITS, int BB, bool PERROW, bool SPLIT>
hipError_t launch_t(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                    const int32_t* zeros, int N, int K, int G, int gsz, int gshift, uint16_t* y,
                    hipStream_t stream) {
  constexpr int R = BB <= 4 ? 2 : 1;
  const int J = (K + codes_per_step<BITS>() - 1) / codes_per_step<BITS>();
  const int Jfull = K / codes_per_step<BITS>();
  const size_t lds = (size_t)J * Unit<BITS>::QUADS * BB * 64 * sizeof(uint4) +
                     (size_t)kWaves * Unit<BITS>::WORDS * 64 * sizeof(uint32_t);
  if (lds > kLdsBudget) return hipErrorNotSupported;
  const int ntiles = (N + kWaves * R - 1) / (kWaves * R);
  const auto kern = qgemv_kernel<BITS, BB, R, PERROW, SPLIT>;
  const int per_cu = resident_blocks(reinterpret_cast<const void*>(kern), kThreads, lds);
  const int cap = device_cu_count() * per_cu;
  const int grid = ntiles < cap ? ntiles : cap;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds, stream, x, packed, scales, zeros, y, N,
                     K, G, gsz, gshift, J, Jfull);
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
