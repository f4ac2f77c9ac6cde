// gemv_kernel.h -- fused dequantize + matrix-vector product, small batches.
//
// y[b][n] = sum_k x[b][k] * deq(packed[n])[k], with deq = (q - z) * s the
// exact value a code stands for on the min-max RTN grid (the stored fp16
// scale and integer zero: BladeLLM model quantization, "Quantization
// algorithms", MinMax; the GGUF type table's weight = code x scale + offset).
// The weights stay low-bit in HBM and are turned back into numbers by the
// GPU's own cores inside the product ([Feature Request] 4bit and 2bit and
// 1bit quantization support: storing 4-bit weights on the GPU and converting
// them at run time); this is the weight-only mode that pays off when memory
// bandwidth is the constraint (BladeLLM model quantization, "Quantization
// modes", weight_only_quant).
//
// Arithmetic.  Per group g of a row, sum_{k in g} x_k (q_k - z) s =
// s * sum_{k in g} x_k (q_k - z).  Each code field is OR-ed, where it sits in
// the packed word, into the fp16 pattern of 2^(10 - p) (p its bit position)
// and one packed subtraction of 2^(10 - p) + z leaves the exact fp16 integer
// q - z: two VALU instructions per pair of codes (unit_decode.h).  The
// products x * (q - z) are exact and are summed in fp32 (matrix cores at
// batch 1 with one group per row, v_dot2_f32_f16 otherwise); the scale
// multiplies the sum of each group (of each unit for grouped rows, of the
// whole row otherwise).  Zero points beyond +-1024, which the subtraction
// cannot take exactly, go through an exact per-code path that enters q - z
// as two fp16 numbers.
//
// Work layout on gfx950:
//  - one persistent workgroup of 16 waves per CU (each workgroup asks for
//    more than half of the CU's LDS, so two never share a CU); x
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
//    below); otherwise v_dot2_f32_f16 accumulates x * (q - z) in fp32; at the
//    end of an item the 64 lanes are summed with DPP permutations into a
//    partial sum in LDS, and the workgroup writes y with coalesced stores,
//    applying the row's scale there (one group per row; grouped rows are
//    scaled per unit).
#pragma once

#include "common.h"
#include "kernels.h"
#include "unit_decode.h"

namespace lowbit {

namespace gemv_detail {

constexpr int kWaves = 16;                 // one 1024-thread workgroup per CU
constexpr int kThreads = kWaves * kWave;
constexpr size_t kLdsBudget = 160 * 1024;   // gfx950 LDS per CU
constexpr size_t kOneWgPerCuLds = kLdsBudget / 2 + 1024;  // above half a CU's LDS
constexpr int kPartMax = 4096;              // fp32 partial sums per round
constexpr size_t kPartMaxMD = 16384;        // same, batch 1 with one group per row
constexpr int kItemsPerWave = 2;            // target work items per wave
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
  const char* row[R];  // first byte of each row's packed words
};

// Separate sums a grouped unit needs: a 3-bit unit's two periods (low /
// high halves) may sit in different groups, and so may a 2-bit unit's two
// 32-code periods when the group size is an odd multiple of 32.
template <int BITS, bool PERROW, bool SPLIT>
constexpr int unit_parts() {
  return (BITS == 3 && !PERROW) || (BITS == 2 && SPLIT) ? 2 : 1;
}

template <int BITS, int BB, int R, bool PERROW, bool SPLIT, bool META>
__global__ __launch_bounds__(kThreads) void qgemv_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros,
    uint16_t* __restrict__ y, int N, int K, int G, int gsz, int gshift, int J, int lgjc,
    int RT) {
  using U = Unit<BITS>;
  constexpr int Q = U::QUADS, W = U::WORDS;
  constexpr int NL = unit_parts<BITS, PERROW, SPLIT>();
  constexpr bool HALVES = BITS == 3 && !PERROW;  // the two halves belong to different groups
  // Batch 1, one group per row: the multiply-accumulate runs on the matrix
  // cores.  Each lane puts its own 8 activations (A operand) and its own 8
  // values q - z (B operand) into v_mfma_f32_16x16x32_f16; the diagonal
  // D[j][j] of the result is then the dot product over lanes j, j+16, j+32,
  // j+48, and the VALU only decodes.  (Off-diagonal entries mix lanes and
  // are ignored.)
  constexpr bool MD = BB == 1 && PERROW;
  // LDS: activations [J][Q][BB][64] | per-wave scratch of the exact path |
  //      partial sums [RT * R rows][BB][JC] | work counter
  extern __shared__ uint4 xs[];

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
  int* counter = reinterpret_cast<int*>(part + RT * R * BB * JC * (MD ? 64 : 1));

  struct Buf {
    uint32_t w[R][W];
    uint16_t s[R][NL];
    int32_t z[R][NL];
  };

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
      t.row[r] = reinterpret_cast<const char*>(packed + (int64_t)min(n0 + r, N - 1) * (row_bytes / 4));
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
    // the K step enters through the descriptor (base + step, the rest of the
    // row as its size: scalar arithmetic), so lanes past the row's end still
    // read zeros and the lanes' offsets stay the same for every step
    const uint32_t step = (uint32_t)j * bytes_per_step<BITS>();
    // zero points (and for grouped rows the scales) before the words, so the
    // wait for the words also covers them
    if constexpr (PERROW) {
      if (j == t.jb) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          uint16_t sb;
          RowParams<META>(scales, zeros, min(n0 + r, N - 1), G).at(0, sb, b.z[r][0]);
        }
      }
    } else {
      const UnitRef u = gemv_unit<BITS>(j, lane, K);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const RowParams<META> rp(scales, zeros, min(n0 + r, N - 1), G);
#pragma unroll
        for (int c = 0; c < NL; ++c) {
          const int kk = BITS == 3 ? (c == 0 ? u.ka : u.kb) : u.ka + 32 * c;
          const bool v = BITS == 3 ? (c == 0 ? u.va : u.vb) : kk < K;
          const int g = v ? group_of(kk, gsz, gshift) : 0;
          rp.at(g, b.s[r][c], b.z[r][c]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const auto rs = rsrc(t.row[r] + step, row_bytes - step);
      if constexpr (BITS == 3) {
        const u3_t va = __builtin_amdgcn_raw_buffer_load_b96(rs, off_a, 0, kSlc);
        const u3_t vb = __builtin_amdgcn_raw_buffer_load_b96(rs, off_b, 0, kSlc);
        b.w[r][0] = va.x;
        b.w[r][1] = va.y;
        b.w[r][2] = va.z;
        b.w[r][3] = vb.x;
        b.w[r][4] = vb.y;
        b.w[r][5] = vb.z;
      } else {
        const u4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, off_a, 0, kSlc);
        b.w[r][0] = v.x;
        b.w[r][1] = v.y;
        b.w[r][2] = v.z;
        b.w[r][3] = v.w;
      }
    }
  };

  float acc[R][BB];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < BB; ++b) acc[r][b] = 0.0f;
  f4_t dacc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) dacc[r] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

  uint32_t mgp[U::NPOS];
  magic_registers<BITS>(mgp);
  // lanes holding an element of the 16x16 accumulator's diagonal (see mfma_diag)
  const bool diag_lane = ((lane & 15) >> 2) == (lane >> 4);
  PConsts<BITS> rowc[R];  // one group per row: the rows' constants (wave-uniform)
  int32_t row_z[R];
  bool rowfast = true;

  auto compute = [&](const Item<R>& t, Buf& b) {
    const int j = t.j;
    const UnitRef u = gemv_unit<BITS>(j, lane, K);
    PConsts<BITS> cc[R][NL];
    HalfParams hp[R][NL];
    bool fast = true;
    if constexpr (PERROW) {
      if (j == t.jb) {
        rowfast = true;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          row_z[r] = (int32_t)uniform((uint32_t)b.z[r][0]);
          rowfast &= row_pconsts<BITS>(row_z[r], rowc[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        cc[r][0] = rowc[r];
        hp[r][0] = HalfParams{0, 0, row_z[r], row_z[r], u.va, u.vb};
      }
      fast = rowfast;
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < NL; ++c) {
          if constexpr (HALVES)  // lo half from period a, hi half from period b
            hp[r][c] = HalfParams{b.s[r][0], b.s[r][1], b.z[r][0], b.z[r][1], u.va, u.vb};
          else
            hp[r][c] = HalfParams{b.s[r][c], b.s[r][c], b.z[r][c], b.z[r][c], u.va, u.vb};
          fast &= make_pconsts<BITS>(hp[r][c], cc[r][c], false);
        }
      fast = __all(fast);
    }
    // the part of slot s (grouped rows: which group sum it belongs to)
    auto part_of = [](int s) { return (BITS == 2 && SPLIT) ? U::cset(s) : 0; };

    const uint4* xj = xs + (int64_t)j * Q * BB * 64 + lane;
    // grouped rows: the unit's sums per part, scaled into acc at the end
    float ts[R][BB][NL];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int bb = 0; bb < BB; ++bb)
#pragma unroll
        for (int c = 0; c < NL; ++c) ts[r][bb][c] = 0.0f;
    // x * d of one slot into the accumulators of row r
    auto accumulate = [&](int r, int s, h2_t d, const uint4 (&xq)[BB], int e) {
#pragma unroll
      for (int bb = 0; bb < BB; ++bb) {
        const uint32_t xv = e == 0 ? xq[bb].x : e == 1 ? xq[bb].y : e == 2 ? xq[bb].z : xq[bb].w;
        const h2_t xh = as_h2(xv);
        if constexpr (PERROW) {
          acc[r][bb] = __builtin_amdgcn_fdot2(d, xh, acc[r][bb], false);
        } else if constexpr (HALVES) {
          ts[r][bb][0] = __builtin_fmaf((float)d.x, (float)xh.x, ts[r][bb][0]);
          ts[r][bb][NL - 1] = __builtin_fmaf((float)d.y, (float)xh.y, ts[r][bb][NL - 1]);
        } else if (NL == 1 || part_of(s) == 0) {  // (no run-time index into registers)
          ts[r][bb][0] = __builtin_amdgcn_fdot2(d, xh, ts[r][bb][0], false);
        } else {
          ts[r][bb][NL - 1] = __builtin_amdgcn_fdot2(d, xh, ts[r][bb][NL - 1], false);
        }
      }
    };

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
          const h8_t bv = __builtin_bit_cast(
              h8_t, make_uint4(as_u32(qz_pair<BITS>(b.w[r], 4 * q + 0, mgp, cc[r][0])),
                               as_u32(qz_pair<BITS>(b.w[r], 4 * q + 1, mgp, cc[r][0])),
                               as_u32(qz_pair<BITS>(b.w[r], 4 * q + 2, mgp, cc[r][0])),
                               as_u32(qz_pair<BITS>(b.w[r], 4 * q + 3, mgp, cc[r][0]))));
          dacc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, dacc[r], 0, 0, 0);
        }
      }
    } else if (fast) {
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
            accumulate(r, s, qz_pair<BITS>(b.w[r], s, mgp, cc[r][NL == 1 ? 0 : part_of(s)]), xq, e);
          }
      }
    } else {
      // Exact per-code path (zero points beyond +-1024): q - z formed in
      // fp32 and entered as two fp16 numbers (its rounding and the
      // remainder).  Kept compact: one slot per loop trip, the unit's words
      // read back from this wave's LDS scratch.
      uint32_t* wsc = slow_scratch + wave * (W * 64);
#pragma unroll
      for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int i = 0; i < W; ++i) wsc[i * 64 + lane] = b.w[r][i];
#pragma unroll 1
        for (int s = 0; s < U::SLOTS; ++s) {
          const HalfParams& h = (HALVES || part_of(s) == 0) ? hp[r][0] : hp[r][NL - 1];
          const float vl = (float)((int)unit_code_lds<BITS>(wsc, lane, U::lo(s)) - h.z_lo);
          const float vh = (float)((int)unit_code_lds<BITS>(wsc, lane, U::hi(s)) - h.z_hi);
          uint16_t hl, ll, hh, lh;
          split_f16(vl, hl, ll);
          split_f16(vh, hh, lh);
          const int q = s >> 2, e = s & 3;
          uint4 xq[BB];
#pragma unroll
          for (int bb = 0; bb < BB; ++bb) xq[bb] = xj[(q * BB + bb) * 64];
          accumulate(r, s, as_h2((uint32_t)hl | ((uint32_t)hh << 16)), xq, e);
          accumulate(r, s, as_h2((uint32_t)ll | ((uint32_t)lh << 16)), xq, e);
        }
      }
    }
    if constexpr (!PERROW) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < NL; ++c) {
          const float sl = h_bits_to_f32(hp[r][c].s_lo);
          const float sh = h_bits_to_f32(hp[r][c].s_hi);
#pragma unroll
          for (int bb = 0; bb < BB; ++bb) {
            if constexpr (HALVES)
              acc[r][bb] += c == 0 ? sl * ts[r][bb][0] : sh * ts[r][bb][NL - 1];
            else
              acc[r][bb] += sl * ts[r][bb][c];
          }
        }
    }

    if (j == t.je - 1) {
      // end of the item
      if constexpr (MD) {
        // The 16 lanes that hold the accumulator's diagonal store their four
        // accumulator values (one LDS write each); the diagonal elements are
        // picked and summed when the round's outputs are written.  An item
        // that took the exact per-code path also has per-lane sums: they are
        // reduced here and added to the diagonal element of lane 0.
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (!rowfast) {
            const float v = wave_sum_dpp(acc[r][0]);
            if (lane == 0) dacc[r][0] += v;
          }
          acc[r][0] = 0.0f;
          if (diag_lane)
            *reinterpret_cast<f4_t*>(part + ((t.tl * R + r) * JC + t.c) * 64 + 4 * (lane & 15)) =
                dacc[r];
          dacc[r] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
      } else {
        // one partial sum per (row, batch row) into LDS
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
          for (int bb = 0; bb < BB; ++bb) {
            float v = acc[r][bb];
            acc[r][bb] = 0.0f;
            v = wave_sum_dpp(v);
            if (lane == 0) part[((t.tl * R + r) * BB + bb) * JC + t.c] = v;
          }
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
        xs[e] = x_entry<BITS>(x + (int64_t)b * K, uu, q, true);
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
    // the round's outputs: sum the K chunks in order (one group per row: times
    // the row's scale), coalesced stores.  The scale of each thread's first
    // output is requested before the barrier, so that its latency overlaps
    // the wait for the workgroup's last items.
    const int row0 = rt0 * R;
    const int nrows = min((rt0 + ntl) * R, N) - row0;
    uint16_t sb_first = 0;
    if constexpr (PERROW) {
      if (tid < nrows * BB) {
        int32_t zz;
        RowParams<META>(scales, zeros, row0 + tid % nrows, G).at(0, sb_first, zz);
      }
    }
    __syncthreads();
    for (int e = tid; e < nrows * BB; e += kThreads) {
      const int bb = e / nrows, rr = e - bb * nrows;
      float v = 0.0f;
      if constexpr (MD) {
        // per K chunk, the 16 diagonal elements: slot j's element is its
        // accumulator value j % 4
        for (int c = 0; c < JC; ++c) {
          const float* pp = part + (rr * JC + c) * 64;
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) v += pp[4 * jj + (jj & 3)];
        }
      } else {
        const float* pp = part + (rr * BB + bb) * JC;
        for (int c = 0; c < JC; ++c) v += pp[c];
      }
      if constexpr (PERROW) {
        uint16_t sb = sb_first;
        int32_t zz;
        if (e != tid) RowParams<META>(scales, zeros, row0 + rr, G).at(0, sb, zz);
        v *= h_bits_to_f32(sb);
      }
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
  // one row per work item: finer items balance the waves better than two
  // rows that share each activation read (measured equal on the largest
  // layer, 4-10% faster on the smaller ones, at batches 1 and 4)
  constexpr int R = 1;
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
  // partial sums per tile: one float per (row, batch row, K chunk), or at
  // batch 1 with one group per row 64 (the diagonal lanes' accumulators)
  constexpr bool MD = BB == 1 && PERROW;
  const size_t fixed = (size_t)J * U::QUADS * BB * 64 * sizeof(uint4) +
                       (size_t)kWaves * U::WORDS * 64 * sizeof(uint32_t) + 16;
  const size_t per_tile = (size_t)R * BB * JC * sizeof(float) * (MD ? 64 : 1);
  const size_t avail = device_lds_per_block() < kLdsBudget ? device_lds_per_block() : kLdsBudget;
  if (fixed + per_tile > avail) return hipErrorNotSupported;
  int RT = MD ? (int)((kPartMaxMD * sizeof(float) < avail - fixed ? kPartMaxMD * sizeof(float)
                                                                   : avail - fixed) /
                      per_tile)
              : kPartMax / (R * BB * JC);
  if (RT > tiles_per_wg) RT = tiles_per_wg;
  if (RT < 1) return hipErrorNotSupported;
  size_t lds = fixed + (size_t)RT * per_tile;
  if (lds > device_lds_per_block() || lds > kLdsBudget) return hipErrorNotSupported;
  // Occupancy bound: the work split gives every workgroup an equal share of
  // the rows and assumes one workgroup per CU.  A request above half of the
  // CU's LDS makes that a hardware guarantee (a second workgroup never fits).
  if (lds < kOneWgPerCuLds && kOneWgPerCuLds <= device_lds_per_block()) lds = kOneWgPerCuLds;
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
