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
//  - one persistent workgroup of 16 waves per CU (the kernel claims the
//    register budget of four waves per SIMD, so two never share a CU); x
//    (all B rows, all K) is staged once per workgroup into LDS, already in
//    the slot order the decode produces;
//  - each workgroup owns an equal, contiguous share of the row tiles (R rows
//    each); its waves draw work items -- a tile, or a K chunk of a tile when
//    there are few tiles per wave -- from a counter in LDS, so a wave that
//    the issue arbiter favours simply takes more items and all waves finish
//    together instead of the youngest ones running alone at the end;
//  - lane l owns units l, l+64, ... of each row, so one load instruction of
//    the wave reads 1 KiB (2/4/8-bit) or 768 B (3-bit) of contiguous packed
//    words; loads are buffer loads with the streaming (slc) cache policy,
//    which measurably raises the HBM read rate on MI355X for data read once,
//    through a per-row resource descriptor whose size is the row's byte
//    count: lanes past the end of the row read zeros instead of touching the
//    next row (the range check applies to the vector offset, so the K step is
//    added there);
//  - the wave walks a flat sequence of (item, K step) iterations, loading the
//    next iteration's words (two register buffers) while decoding the
//    current one, so HBM reads stay in flight across item boundaries;
//  - batch 1 with one group per row multiplies on the matrix cores (see
//    below); otherwise v_dot2_f32_f16 accumulates x * deq in fp32; at the end
//    of an item the 64 lanes are summed with DPP permutations into a partial
//    sum in LDS, and the workgroup writes y with coalesced stores;
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

constexpr int kWaves = 16;                 // one 1024-thread workgroup per CU
constexpr int kThreads = kWaves * kWave;
constexpr size_t kLdsBudget = 160 * 1024;   // gfx950 LDS per CU
constexpr int kPartMax = 4096;              // fp32 partial sums per round
constexpr int kItemsPerWave = 4;            // target work items per wave
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

// One work item: R consecutive rows (a "tile") of this workgroup's current
// round, over K steps [jb, je) (K chunk c of 2^lgjc), with the buffer
// descriptors of its rows.
template <int R>
struct Item {
  int i;       // item number; i >= nit means no more work
  int tl;      // tile index inside the round
  int c;       // K chunk
  int jb, je;  // K steps of the chunk
  int j;       // K step being loaded / computed
  __amdgpu_buffer_rsrc_t rs[R];
};

template <int BITS, int BB, int R, bool PERROW, bool SPLIT, bool META>
__global__ __launch_bounds__(kThreads) void qgemv_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros,
    uint16_t* __restrict__ y, int N, int K, int G, int gsz, int gshift, int J, int lgjc,
    int RT) {
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
  // LDS: activations [J][Q][BB][64] | per-wave slow-path scratch |
  //      partial sums [RT * R rows][BB][JC] | work counter
  extern __shared__ uint4 xs[];

  // Claim the whole register budget of four waves per SIMD, so that two of
  // these 16-wave workgroups can never share a CU (the work split below
  // assumes one workgroup per CU).
  asm volatile("" ::: "v127");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t row_bytes = (uint32_t)K * BITS / 8;
  // per-lane byte offsets of the lane's unit inside one K step
  const uint32_t off_a = BITS == 3 ? 12u * lane : 16u * lane;
  const uint32_t off_b = off_a + 768u;

  // This workgroup's tiles: an equal share of all of them, in rounds of at
  // most RT tiles (bounded by the partial-sum space).
  const int T = (N + R - 1) / R;
  const int nwg = (int)gridDim.x, wg = (int)blockIdx.x;
  const int tbase = T / nwg, textra = T % nwg;
  const int t0 = wg * tbase + min(wg, textra);
  const int t1 = t0 + tbase + (wg < textra ? 1 : 0);

  const int JC = 1 << lgjc;
  const int entries = J * Q * BB * 64;
  uint32_t* slow_scratch = reinterpret_cast<uint32_t*>(xs + entries);
  float* part = reinterpret_cast<float*>(slow_scratch + kWaves * W * 64);
  int* counter = reinterpret_cast<int*>(part + RT * R * BB * JC);

  struct Buf {
    uint32_t w[R][W];
    uint16_t s[R][NL];
    int32_t z[R][NL];
  };

  // META: `scales` holds the compact words (4 bytes per group) and the
  // zeros descriptor is empty
  const auto srs =
      rsrc(scales, (uint32_t)min((int64_t)N * G * (META ? 4 : 2), (int64_t)0x7fffffff));
  const auto zrs = rsrc(zeros, META ? 0u : (uint32_t)min((int64_t)N * G * 4, (int64_t)0x7fffffff));
  int rt0 = t0;  // first tile of the current round
  int nit = 0;   // items of the current round

  auto make_item = [&](int i) {
    Item<R> t;
    t.i = i;
    t.tl = i >> lgjc;
    t.c = i & (JC - 1);
    t.jb = (t.c * J) >> lgjc;
    t.je = ((t.c + 1) * J) >> lgjc;
    t.j = t.jb;
    const int n0 = (rt0 + t.tl) * R;
#pragma unroll
    for (int r = 0; r < R; ++r)
      t.rs[r] = rsrc(packed + (int64_t)min(n0 + r, N - 1) * (row_bytes / 4), row_bytes);
    return t;
  };
  // Next (item, K step) of this wave: the next step of the same item, else a
  // fresh item from the workgroup's counter (an LDS atomic by lane 0).
  auto next_of = [&](const Item<R>& t) {
    if (t.j + 1 < t.je) {
      Item<R> u = t;
      ++u.j;
      return u;
    }
    int v = 0;
    if (lane == 0) v = atomicAdd(counter, 1);
    v = __builtin_amdgcn_readfirstlane(v);
    return make_item(v < nit ? v : nit);
  };

  auto load = [&](const Item<R>& t, Buf& b) {
    const int n0 = (rt0 + t.tl) * R;
    const int j = t.j;
    const uint32_t step = (uint32_t)j * bytes_per_step<BITS>();
    const uint32_t va_off = off_a + step, vb_off = off_b + step;
    UnitRef u;
    if constexpr (!PERROW) u = gemv_unit<BITS>(j, lane, K);
    // scale / zero loads first: a wait for this step's words then also
    // covers them, whatever the number of loads issued after
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = min(n0 + r, N - 1);
      if constexpr (PERROW) {
        if (j == t.jb) {
          // vector (buffer) loads on purpose: a scalar load would share the
          // lgkm counter with the LDS activation reads, and every wait on
          // those would then also wait for this prefetch to come from HBM
          const uint32_t nn = (uint32_t)n + 0u * (uint32_t)lane;
          if constexpr (META) {
            const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(srs, 4u * nn, 0, 0);
            b.s[r][0] = (uint16_t)v;
            b.z[r][0] = (int32_t)v >> 16;
          } else {
            b.s[r][0] = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(srs, 2u * nn, 0, 0);
            b.z[r][0] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(zrs, 4u * nn, 0, 0);
          }
        }
      } else {
        const RowParams<META> rp(scales, zeros, n, G);
#pragma unroll
        for (int c = 0; c < NL; ++c) {
          const int kk = BITS == 3 ? (c == 0 ? u.ka : u.kb) : u.ka + 32 * c;
          const bool v = BITS == 3 ? (c == 0 ? u.va : u.vb) : u.va;
          const int g = v ? group_of(kk, gsz, gshift) : 0;
          rp.at(g, b.s[r][c], b.z[r][c]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const auto rs = t.rs[r];
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
    }
  };

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

  auto compute = [&](const Item<R>& t, Buf& b) {
    const int j = t.j;
    const UnitRef u = gemv_unit<BITS>(j, lane, K);
    HalfParams hp[R][NC];
    Consts<BITS> cc[R][NC];
    bool fast = true;
    if constexpr (PERROW) {
      if (j == t.jb) {
        rowfast = true;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          rows_s[r] = (uint16_t)uniform(b.s[r][0]);
          rows_z[r] = (int32_t)uniform((uint32_t)b.z[r][0]);
          HalfParams h{rows_s[r], rows_s[r], rows_z[r], rows_z[r], true, true};
          rowfast &= make_consts<BITS, false>(h, rowc[r]);
          // Positions past the end of the row (last K step of a ragged row)
          // are decoded from zero words without masking: their activations
          // are staged as zeros, so only a finite decode is needed there,
          // which |q - z| * s <= 15 * s < 65504 guarantees (8-bit codes:
          // the fast-path bounds z <= 255, s < 256).
          rowfast &= rows_s[r] < 0x6C00u;  // s < 4096
#pragma unroll
          for (int i = 0; i < U::NPOS; ++i) {
            rowc[r].hz[i] = as_h2(uniform(as_u32(rowc[r].hz[i])));
            rowc[r].hs[i] = as_h2(uniform(as_u32(rowc[r].hs[i])));
          }
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) cc[r][0] = rowc[r];
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
      // all activation quads of the step first: one LDS wait per step
      uint4 xq[Q];
#pragma unroll
      for (int q = 0; q < Q; ++q) xq[q] = xj[q * 64];
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const h8_t av = __builtin_bit_cast(h8_t, xq[q]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          h2_t d[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int s = quad_slot<BITS, POS>(q, e);
            const int c = NC == 1 ? 0 : U::cset(s);
            d[e] = fast_pair<BITS, POS>(b.w[r], s, cc[r][c], mg);
          }
          const h8_t bv = __builtin_bit_cast(
              h8_t, make_uint4(as_u32(d[0]), as_u32(d[1]), as_u32(d[2]), as_u32(d[3])));
          const int a = POS ? U::pidx(U::pos(quad_slot<BITS, POS>(q, 0))) : 0;
          dacc[r][MD ? a : 0] =
              __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, dacc[r][MD ? a : 0], 0, 0, 0);
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
          const HalfParams h =
              PERROW ? HalfParams{rows_s[r], rows_s[r], rows_z[r], rows_z[r], u.va, u.vb}
                     : c == 0 ? hp[r][0] : hp[r][NC - 1];
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

    if (j == t.je - 1) {
      // end of the item: one partial sum per (row, batch row) into LDS
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
          if (lane == 0) part[((t.tl * R + r) * BB + bb) * JC + t.c] = v;
#pragma unroll
          for (int a = 0; a < NA; ++a) acc[r][bb][a] = 0.0f;
        }
      }
    }
  };

  Buf bufA, bufB;
  for (bool first = true; rt0 < t1; rt0 += RT, first = false) {
    const int ntl = min(RT, t1 - rt0);
    nit = ntl * JC;
    // items 0 .. kWaves-1 go to waves 0 .. kWaves-1; the rest are claimed
    Item<R> cur = make_item(wave < nit ? wave : nit);
    // the first weights are requested before the activations are staged, so
    // their HBM latency overlaps the staging
    if (cur.i < nit) load(cur, bufA);
    if (tid == 0) *counter = kWaves;
    if (first) {
      for (int e = tid; e < entries; e += kThreads) {
        const int l = e & 63;
        int rest = e >> 6;
        const int b = rest % BB;
        rest /= BB;
        const int q = rest % Q;
        const int jj = rest / Q;
        const UnitRef uu = gemv_unit<BITS>(jj, l, K);
        xs[e] = MD ? x_entry_ordered<BITS, POS>(x + (int64_t)b * K, uu, q)
                   : x_entry<BITS>(x + (int64_t)b * K, uu, q, true);
      }
    }
    __syncthreads();

    // Two-deep software pipeline: the loads of the next (item, K step) are
    // issued before the current one is decoded.
    // The prefetch is issued even past the last item (its rows are clamped
    // to valid memory and the words are never used): an unconditional load
    // keeps the wait before each decode at "all but the newest loads done".
    while (cur.i < nit) {
      Item<R> nx = next_of(cur);
      load(nx, bufB);
      compute(cur, bufA);
      cur = nx;
      if (cur.i >= nit) break;
      nx = next_of(cur);
      load(nx, bufA);
      compute(cur, bufB);
      cur = nx;
    }
    __syncthreads();

    // the round's outputs: sum the K chunks in order, coalesced stores
    const int row0 = rt0 * R;
    const int nrows = min((rt0 + ntl) * R, N) - row0;
    for (int e = tid; e < nrows * BB; e += kThreads) {
      const int bb = e / nrows, rr = e - bb * nrows;
      const float* pp = part + (rr * BB + bb) * JC;
      float v = 0.0f;
      for (int c = 0; c < JC; ++c) v += pp[c];
      y[(int64_t)bb * N + row0 + rr] = f32_to_h_bits(v);
    }
    __syncthreads();  // partial sums and counter are reused by the next round
  }
}

template <int BITS, int BB, bool PERROW, bool SPLIT, bool META>
hipError_t launch_t(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                    const int32_t* zeros, int N, int K, int G, int gsz, int gshift, uint16_t* y,
                    hipStream_t stream) {
  using U = Unit<BITS>;
  // two rows per wave where the accumulators leave room for a second row
  constexpr int NA = PERROW ? 1 : U::NPOS;
  constexpr int R = (BB <= 4 && BB * NA <= 16) ? 2 : 1;
  const int J = (K + codes_per_step<BITS>() - 1) / codes_per_step<BITS>();
  const int T = (N + R - 1) / R;
  const int cus = device_cu_count();
  const int nwg = T < cus ? T : cus;
  const int tiles_per_wg = (T + nwg - 1) / nwg;
  // K chunks per tile (a power of two, at most J): enough work items that
  // every wave draws several
  int lgjc = 0;
  while ((tiles_per_wg << lgjc) < kItemsPerWave * kWaves && (2 << lgjc) <= J) ++lgjc;
  const int JC = 1 << lgjc;
  int RT = kPartMax / (R * BB * JC);
  if (RT > tiles_per_wg) RT = tiles_per_wg;
  if (RT < 1) return hipErrorNotSupported;
  const size_t lds = (size_t)J * U::QUADS * BB * 64 * sizeof(uint4) +
                     (size_t)kWaves * U::WORDS * 64 * sizeof(uint32_t) +
                     (size_t)RT * R * BB * JC * sizeof(float) + 16;
  if (lds > device_lds_per_block() || lds > kLdsBudget) return hipErrorNotSupported;
  const auto kern = qgemv_kernel<BITS, BB, R, PERROW, SPLIT, META>;
  if (lds > 64 * 1024) {
    // above the default limit: raise it (once per device) to the largest
    // request this kernel can make
    const int cap = (int)(device_lds_per_block() < kLdsBudget ? device_lds_per_block() : kLdsBudget);
    const hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(kern), cap);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(kThreads), lds, stream, x, packed, scales, zeros, y, N,
                     K, G, gsz, gshift, J, lgjc, RT);
  return hipGetLastError();
}

template <int BITS, bool PERROW, bool SPLIT, bool META>
hipError_t launch_bits(int B, const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                       const int32_t* zeros, int N, int K, int G, int gsz, int gshift,
                       uint16_t* y, hipStream_t stream) {
#define LOWBIT_GEMV_CASE(bb)                                                                  \
  case bb:                                                                                    \
    return launch_t<BITS, bb, PERROW, SPLIT, META>(x, packed, scales, zeros, N, K, G, gsz,  \
                                                   gshift, y, stream);
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

// Per-width entry (instantiated in gemv2.hip, gemv3.hip, gemv4.hip,
// gemv8.hip).  meta: `scales` holds compact words (see RowParams), `zeros`
// is unused.
template <int BITS, bool META>
hipError_t launch_qgemv_layout(const uint16_t* x, int B, const uint32_t* packed,
                               const uint16_t* scales, const int32_t* zeros, int N, int K, int G,
                               int gsz, int gshift, uint16_t* y, hipStream_t stream) {
  using namespace gemv_detail;
  if (G == 1)
    return launch_bits<BITS, true, false, META>(B, x, packed, scales, zeros, N, K, G, gsz, gshift,
                                                y, stream);
  if constexpr (BITS == 2) {
    if (gsz % 64 != 0)
      return launch_bits<2, false, true, META>(B, x, packed, scales, zeros, N, K, G, gsz, gshift,
                                               y, stream);
  }
  return launch_bits<BITS, false, false, META>(B, x, packed, scales, zeros, N, K, G, gsz, gshift,
                                               y, stream);
}

template <int BITS>
hipError_t launch_qgemv_bits(const uint16_t* x, int B, const uint32_t* packed,
                             const uint16_t* scales, const int32_t* zeros, int N, int K,
                             int G, int gsz, int gshift, bool meta, uint16_t* y,
                             hipStream_t stream) {
  return meta ? launch_qgemv_layout<BITS, true>(x, B, packed, scales, zeros, N, K, G, gsz, gshift,
                                                y, stream)
              : launch_qgemv_layout<BITS, false>(x, B, packed, scales, zeros, N, K, G, gsz,
                                                 gshift, y, stream);
}

}  // namespace lowbit
