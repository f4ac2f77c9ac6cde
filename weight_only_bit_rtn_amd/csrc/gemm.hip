// gemm.hip -- fused dequantize + small-batch matrix product on the fp16
// matrix cores (v_mfma_f32_16x16x32_f16 of gfx950).
//
// y[b][n] = sum_k x[b][k] * deq(packed[n])[k] with deq = (q - z) * s, the
// exact value of each code, the same contract as the matrix-vector kernel;
// this one is for batches where the product is a real dense contraction (the
// matrix cores do the multiply-adds, the vector ALUs only decode).  The
// weights are decoded from their low-bit form by the GPU's own cores at run
// time ([Feature Request] 4bit and 2bit and 1bit quantization support) and go
// from registers straight into the MFMA B operand: as the exact fp16
// integers q - z, with the scale applied to the fp32 sums (one group per row,
// and groups that hold every MFMA's codes whole), or else as (q - z) * s
// split into an fp16 value and its exact fp16 remainder, two MFMAs.
//
// Work layout (one persistent workgroup of 8 waves per CU):
//  - the weight rows are cut into groups of 16 (the MFMA's 16 columns); each
//    workgroup owns an equal, contiguous share of the groups and walks them
//    in rounds of at most 8 groups;
//  - in a round, wave w works on row group (w % RG) and K part (w / RG): with
//    RG groups in the round, KP = 8 / RG waves split K between them, so few
//    groups per CU still keep all waves busy;
//  - K is walked in tiles; a tile holds, for every K part, four lane groups
//    times NW units (see unit_decode.h) per row;  lane l decodes row (l % 16)
//    of its group, lane group h = l / 16 takes NW of the part's units: NW
//    consecutive ones (2-, 3-, 4-bit), or runs of two interleaved with the
//    other lane groups' runs (8-bit, one 128-byte line per row and load);
//  - x for the tile (all batch rows, zero past K and past B) is staged in
//    LDS, double buffered, already in the decode's slot order, so one MFMA A
//    operand is one 16-byte LDS read; the next tile's weights and x are
//    loaded while the current tile is multiplied;
//  - each wave keeps 16 x (16 * BT) fp32 accumulators in registers over all
//    of K; at the end of a round the K parts meet in LDS and are summed in a
//    fixed order (deterministic), and y is written with coalesced stores.
//  - the contraction order inside one 32-long MFMA step is the slot order, a
//    permutation of k applied identically to both operands.
#include "common.h"
#include "kernels.h"
#include "unit_decode.h"

namespace lowbit {

namespace {

constexpr int kWaves = 8;  // two per SIMD: each wave may hold 256 registers
constexpr int kThreads = kWaves * kWave;
constexpr int kTileK = 512;  // k extent of one step: its activations are one LDS buffer

typedef uint32_t u3_t __attribute__((ext_vector_type(3)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Group layout of the scales and zeros: one per row, power-of-two groups
// (group index by a shift), any other group size (a division), or
// power-of-two groups at least as long as a lane's run of units (2-, 4- and
// 8-bit): then the run shares one group, loaded once per run.
enum GroupMode { kPerRow = 0, kPow2Groups = 1, kAnyGroups = 2, kWideGroups = 3 };

// Scales and zeros of constant set c of unit u: its low and high halves'
// groups (a position past the row end takes the last group of the row, a
// finite scale; its weight meets a zero activation).
template <int BITS, int GM, bool META>
__device__ __forceinline__ HalfParams params_at(const RowParams<META>& rp, int gsz, int gshift,
                                                const UnitRef& u, int c, int K) {
  int kl, kh;
  if constexpr (BITS == 3) {
    kl = u.ka;
    kh = u.kb;
  } else if constexpr (BITS == 2) {
    kl = kh = u.ka + 32 * c;
  } else {
    kl = kh = u.ka;
  }
  const uint32_t cl = (uint32_t)min(kl, K - 1), ch = (uint32_t)min(kh, K - 1);
  const uint32_t gl = GM == kAnyGroups ? cl / (uint32_t)gsz : cl >> gshift;
  const uint32_t gh = GM == kAnyGroups ? ch / (uint32_t)gsz : ch >> gshift;
  HalfParams hp;
  rp.at((int)gl, hp.s_lo, hp.z_lo);
  rp.at((int)gh, hp.s_hi, hp.z_hi);
  hp.v_lo = kl < K;
  hp.v_hi = kh < K;
  return hp;
}

template <int BITS, int BT, int GM, bool META, bool SS>
__global__ __launch_bounds__(kThreads) void qgemm_kernel(
    const uint16_t* __restrict__ x, int B, const uint32_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros,
    uint16_t* __restrict__ y, int N, int K, int G, int gsz, int gshift, int pstage) {
  using U = Unit<BITS>;
  constexpr int Q = U::QUADS, W = U::WORDS, NC = U::NCONST;
  constexpr bool PERROW = GM == kPerRow;
  constexpr int BP = 16 * BT;               // batch rows per pass (padded)
  constexpr int UT = kTileK / U::CODES;     // units (3-bit: period pairs) per step
  constexpr int NWMAX = UT / 4;             // units per lane and step (one K part)
  constexpr int E = 2 * BT;                 // activation entries per thread and step
  constexpr int XBUF = kTileK * BP * 2 / 16;  // 16-byte entries of one activation buffer
  static_assert(XBUF == E * kThreads, "one step's activations are E entries per thread");
  // 8-bit lanes take runs of two consecutive units (others single units)
  constexpr bool kRuns2 = BITS == 8;
  // exact dequantized values in two MFMA operands (hi + lo), for group
  // layouts whose groups do not hold every MFMA's units whole
  constexpr bool DIRECT = GM == kPow2Groups || GM == kAnyGroups;
  // LDS: two activation tiles (later the partial sums), then per-wave scratch
  // of the exact decode path, then (wide groups, when the host asks for it)
  // each wave's copy of its 16 rows' scales and zeros
  extern __shared__ uint4 lds[];
  uint32_t* slow_scratch = reinterpret_cast<uint32_t*>(lds + 2 * XBUF);
  // staged parameters, in 32-bit words: a row's G scales (fp16 pairs) at
  // stride ssw, its G zeros (or compact words) at stride zsw; the padding
  // spreads the 16 rows of one read over the banks
  // (batch tiles of 64 rows leave too little LDS, and the code would cost
  // them registers, so they never stage)
  constexpr bool kStage = GM == kWideGroups && BT <= 2;
  // Batch tiles of 64 rows have no room for a round's copy; instead, in the
  // SS variant (the host's choice: wide groups of exactly a run's span, K in
  // whole steps, 16-byte aligned arrays, every round of every workgroup with
  // at least five row groups, hence one K part), each step's parameters of
  // all the round's rows are staged next to the step's activations, double
  // buffered: one cooperative load per wave and step instead of two loads
  // per lane.  Layout: 8 words per row, the scales (fp16 pairs) from word 0,
  // the zeros (or compact words) from word 4.
  static_assert(!SS || (GM == kWideGroups && BT == 4), "step staging: 64-row tiles, wide groups");
  constexpr bool kStepStage = SS;
  uint32_t* const ps = slow_scratch + kWaves * W * 64;
  const int ssw = G / 2 + 2, zsw = G + 4;
  const int pww = META ? 16 * zsw : 16 * (ssw + zsw);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, h = lane >> 4;
  const uint32_t row_bytes = (uint32_t)K * BITS / 8;
  const int row_words = (int)(row_bytes / 4);
  const int units_per_row = BITS == 3 ? K / 32 : (K + U::CODES - 1) / U::CODES;  // 3-bit: periods
  const auto xrs = make_rsrc(x, (uint32_t)((int64_t)B * K * 2));

  const int NG = (N + 15) / 16;
  const int nwg = (int)gridDim.x, wg = (int)blockIdx.x;
  const int gb = NG / nwg, ge = NG % nwg;
  const int g0 = wg * gb + min(wg, ge);
  const int g1 = g0 + gb + (wg < ge ? 1 : 0);

  uint32_t mgp[U::NPOS];
  magic_registers<BITS>(mgp);

  for (int gr0 = g0; gr0 < g1; gr0 += kWaves) {
    const int RG = min(kWaves, g1 - gr0);
    // K parts: the largest power of two that fits both the waves and the step
    int KP = 1;
    while (KP * 2 * RG <= kWaves && KP * 2 <= NWMAX) KP *= 2;
    const int NW = NWMAX / KP;  // units per lane and step
    const int T = BITS == 3 ? (units_per_row + 2 * UT - 1) / (2 * UT)
                            : (units_per_row + UT - 1) / UT;
    const bool active = wave < RG * KP;
    const int gl = wave % RG, kp = wave / RG;
    const int grp = gr0 + gl;
    const int n = min(16 * grp + i16, N - 1);
    const int rows_here = max(0, min(16, N - 16 * grp));
    // buffer descriptor over this wave's 16 rows (rows past N read zeros);
    // its parts are made explicitly wave-uniform, or the compiler would keep
    // it in vector registers and loop over its distinct values at every load
    const uint64_t rbase = reinterpret_cast<uint64_t>(packed + (int64_t)16 * min(grp, NG - 1) * row_words);
    const uint32_t rlo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)rbase);
    const uint32_t rhi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(rbase >> 32));
    const uint32_t rbytes = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)min((int64_t)rows_here * row_bytes, (int64_t)0x7fffffff));
    const auto rs = make_rsrc(reinterpret_cast<const void*>(((uint64_t)rhi << 32) | rlo), rbytes);
    const uint32_t row_off = (uint32_t)i16 * row_bytes;
    // META: `scales` holds compact words (see RowParams), `zeros` is unused
    const RowParams<META> rp(scales, zeros, n, G);

    // Wide groups: the wave copies its 16 rows' scales and zeros into LDS
    // once per round (one contiguous read per row), so the steps read them
    // from LDS instead of issuing one more global load per parameter array
    // and step; rows past N take row N - 1, whose outputs are not written.
    // The host asks for this only when G is a multiple of 8, the arrays are
    // 16-byte aligned and the copy fits the LDS.
    uint32_t* pw = slow_scratch + kWaves * W * 64 + wave * pww;
    if constexpr (kStage) {
      if (pstage) {
        const int sc = META ? G / 4 : G / 8;  // 16-byte chunks of a row's first array
        for (int e = lane; e < 16 * sc; e += 64) {
          const int r = e / sc, c = e - r * sc;
          const int64_t nr = min(16 * grp + r, N - 1);
          const uint4 v = *reinterpret_cast<const uint4*>(scales + (nr * G + (META ? 4 : 8) * c) * (META ? 2 : 1));
          uint32_t* d = pw + r * (META ? zsw : ssw) + 4 * c;
          d[0] = v.x, d[1] = v.y, d[2] = v.z, d[3] = v.w;
        }
        if constexpr (!META) {
          const int zc = G / 4;
          for (int e = lane; e < 16 * zc; e += 64) {
            const int r = e / zc, c = e - r * zc;
            const int64_t nr = min(16 * grp + r, N - 1);
            const int4 v = *reinterpret_cast<const int4*>(zeros + nr * G + 4 * c);
            *reinterpret_cast<int4*>(pw + 16 * ssw + r * zsw + 4 * c) = v;
          }
        }
        // other lanes of this wave read these rows: order the LDS writes
        // before their reads (a wave-scope release / acquire pair around a
        // wave barrier; no workgroup barrier is needed, the slice is the
        // wave's own)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }

    // per-row constants (one group per row): computed once per round; the
    // row's scale multiplies the finished sum
    PConsts<BITS> rowc;
    bool rowfast = true;
    float row_scale = 0.0f;
    HalfParams rowp{};
    if constexpr (PERROW) {
      uint16_t s0;
      int32_t z0;
      rp.at(0, s0, z0);
      rowp = HalfParams{s0, s0, z0, z0, true, true};
      rowfast = make_pconsts<BITS>(rowp, rowc, false);
      row_scale = h_bits_to_f32(s0);
    }

    f4_t acc[BT];
#pragma unroll
    for (int bt = 0; bt < BT; ++bt) acc[bt] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // unit ug of step t (4-bit / 2-bit: CODES codes; 3-bit: two periods)
    auto unit_at = [&](int t, int ug) {
      UnitRef u;
      if constexpr (BITS == 3) {
        const int pa = 2 * UT * t + ug, pb = pa + UT;
        u.ka = 32 * pa;
        u.kb = 32 * pb;
      } else {
        u.ka = U::CODES * (UT * t + ug);
        u.kb = u.ka;
      }
      u.va = u.ka < K;
      u.vb = u.kb < K;
      return u;
    };
    // Units of a K part (4 * NW of them) go to the four lanes of a row in
    // runs of RN: lane group h takes units 4 * RN * (u / RN) + RN * h +
    // u % RN, and a lane's run shares its group constants.  2-, 3- and 4-bit
    // lanes take one run of NW consecutive units (one group per step for
    // wide groups); 8-bit lanes, with twice the bytes per code, take runs of
    // two, so that one load instruction of the wave reads each row's eight
    // consecutive units, one 128-byte line per row, instead of four lines.
    const int RN = kRuns2 && NW >= 2 ? 2 : 1;
    // wide groups: runs per lane and step, and whether a step's groups load
    // as vectors (see load_w)
    constexpr int NVMAX = kRuns2 ? NWMAX / 2 : NWMAX;
    const bool wide_vec = NW == NWMAX && gsz == 4 * RN * U::CODES && G % NVMAX == 0;
    // every wave of the round walks the same step (one K part): stage its
    // parameters cooperatively (see kStepStage)
    constexpr bool sstage = kStepStage;  // (one K part: the host's condition)
    // Step t's parameters: waves 0-1 load the scales (compact words) of the
    // round's rows 64 (w % 2) .. 64 (w % 2) + 63, waves 2-3 the zeros, one
    // 16-byte load per lane (the groups of the step); every other wave loads
    // from an empty descriptor (zeros, no memory traffic), so each wave
    // issues the same loads on every path.
    const int prole = META ? (wave < 2 ? 0 : 2) : (wave < 4 ? wave >> 1 : 2);  // 0 s, 1 z, 2 none
    const int prow = 64 * (wave & 1) + lane;
    uint4 pr = make_uint4(0u, 0u, 0u, 0u);
    auto fetch_p = [&](int t) {
      const bool on = sstage && prole < 2 && prow < RG * 16;
      const uint32_t esz = prole == 0 && !META ? 2u : 4u;
      const void* base = prole == 0 ? static_cast<const void*>(scales)
                                    : static_cast<const void*>(zeros);
      const uint64_t bb = reinterpret_cast<uint64_t>(base);
      const uint32_t blo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)bb);
      const uint32_t bhi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(bb >> 32));
      const uint32_t bytes = (uint32_t)__builtin_amdgcn_readfirstlane(
          (int)(prole < 2 ? min((int64_t)N * G * esz, (int64_t)0x7fffffff) : 0));
      const auto prs = make_rsrc(reinterpret_cast<const void*>(((uint64_t)bhi << 32) | blo), bytes);
      const int64_t nr = min(16 * gr0 + prow, N - 1);
      const uint32_t off = on ? (uint32_t)((nr * G + (int64_t)t * NVMAX) * esz) : 0u;
      const u4_t v = __builtin_amdgcn_raw_buffer_load_b128(prs, off, 0, 0);
      pr = make_uint4(v.x, v.y, v.z, v.w);
    };
    auto store_p = [&](int buf) {
      if (!(sstage && prole < 2 && prow < RG * 16)) return;
      uint32_t* d = ps + buf * 1024 + 8 * prow;
      if (prole == 0 && !META) {
        d[0] = pr.x;
        if constexpr (NVMAX == 4) d[1] = pr.y;
      } else {
        d[4] = pr.x;
        d[5] = pr.y;
        if constexpr (NVMAX == 4) {
          d[6] = pr.z;
          d[7] = pr.w;
        }
      }
    };
    // index of the first unit of u's run (its group constants live there;
    // a compile-time index after unrolling)
    auto run_start = [](int u) { return kRuns2 ? (u & ~1) : u; };
    auto part_unit = [&](int u) { return 4 * RN * (u / RN) + RN * h + u % RN; };
    auto my_unit = [&](int t, int u) { return unit_at(t, kp * 4 * NW + part_unit(u)); };

    struct WBuf {
      uint32_t w[NWMAX][W];
      // grouped layouts: the units' scales and zeros (wide groups: one set
      // per run, kept at the run's first index)
      HalfParams hp[PERROW ? 1 : NWMAX][NC];
    };
    // Weight loads of step t: always NWMAX units per lane (clamped to the row,
    // unused ones discarded), so every step issues the same number of loads.
    auto load_w = [&](int t, WBuf& b) {
#pragma unroll
      for (int u = 0; u < NWMAX; ++u) {
        const UnitRef ur = my_unit(t, u < NW ? u : 0);
        if constexpr (BITS == 3) {
          const int pa = min(ur.ka >> 5, units_per_row - 1), pb = min(ur.kb >> 5, units_per_row - 1);
          const u3_t va = __builtin_amdgcn_raw_buffer_load_b96(rs, row_off + 12u * pa, 0, 2);
          const u3_t vb = __builtin_amdgcn_raw_buffer_load_b96(rs, row_off + 12u * pb, 0, 2);
          b.w[u][0] = va.x;
          b.w[u][1] = va.y;
          b.w[u][2] = va.z;
          b.w[u][3] = vb.x;
          b.w[u][4] = vb.y;
          b.w[u][5] = vb.z;
        } else {
          const int gu = min(ur.ka / U::CODES, units_per_row - 1);
          const u4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, row_off + 16u * gu, 0, 2);
          b.w[u][0] = v.x;
          b.w[u][1] = v.y;
          b.w[u][2] = v.z;
          b.w[u][3] = v.w;
        }
        // grouped layouts: this unit's scales and zeros come with its words
        // (positions past the row end take the row's last group)
        if constexpr (GM == kPow2Groups || GM == kAnyGroups) {
#pragma unroll
          for (int c = 0; c < NC; ++c)
            b.hp[u][c] = params_at<BITS, GM, META>(rp, gsz, gshift, ur, c, K);
        }
      }
      if constexpr (GM == kWideGroups) {
        if constexpr (!sstage) {
          // One group per run of units.  A full step (K split in one part)
          // whose group size is exactly the unit span takes consecutive groups
          // g0 .. g0 + NVMAX - 1 for its runs, g0 a multiple of NVMAX: one
          // vector load per parameter array instead of one load per run
          // (measured 5-10% faster at batches 16 and 32 on scale/zero arrays).
          // Otherwise, and for the row's last step, the groups load per run.
          const int g0 = min(my_unit(t, 0).ka, K - 1) >> gshift;
          if (wide_vec && g0 + NVMAX <= G) {
            uint16_t sv[NVMAX];
            int32_t zv[NVMAX];
            if (kStage && pstage) {
              uint32_t wv[NVMAX];
              if constexpr (META) {
                const uint32_t* mp = pw + i16 * zsw + g0;
                if constexpr (NVMAX == 4) {
                  const uint4 v = *reinterpret_cast<const uint4*>(mp);
                  wv[0] = v.x, wv[1] = v.y, wv[2] = v.z, wv[3] = v.w;
                } else {
                  const uint2 v = *reinterpret_cast<const uint2*>(mp);
                  wv[0] = v.x, wv[1] = v.y;
                }
#pragma unroll
                for (int i = 0; i < NVMAX; ++i) zv[i] = (int32_t)wv[i] >> 16;
              } else {
                const uint32_t* sp = pw + i16 * ssw + g0 / 2;
                const int32_t* zp = reinterpret_cast<const int32_t*>(pw + 16 * ssw + i16 * zsw + g0);
                if constexpr (NVMAX == 4) {
                  const uint2 v = *reinterpret_cast<const uint2*>(sp);
                  wv[0] = v.x, wv[1] = v.x >> 16, wv[2] = v.y, wv[3] = v.y >> 16;
                  const int4 z4 = *reinterpret_cast<const int4*>(zp);
                  zv[0] = z4.x, zv[1] = z4.y, zv[2] = z4.z, zv[3] = z4.w;
                } else {
                  const uint32_t v = *sp;
                  wv[0] = v, wv[1] = v >> 16;
                  const int2 z2 = *reinterpret_cast<const int2*>(zp);
                  zv[0] = z2.x, zv[1] = z2.y;
                }
              }
#pragma unroll
              for (int i = 0; i < NVMAX; ++i) sv[i] = (uint16_t)wv[i];
            } else {
              rp.template at_vec<NVMAX>(g0, sv, zv);
            }
#pragma unroll
            for (int u = 0; u < NWMAX; ++u)
              if (run_start(u) == u) {
                const int i = kRuns2 ? u >> 1 : u;
#pragma unroll
                for (int c = 0; c < NC; ++c)
                  b.hp[u][c] = HalfParams{sv[i], sv[i], zv[i], zv[i], true, true};
              }
          } else {
#pragma unroll
            for (int u = 0; u < NWMAX; ++u)
              if (run_start(u) == u) {
                const UnitRef ur = my_unit(t, u < NW ? u : 0);
#pragma unroll
                for (int c = 0; c < NC; ++c)
                  b.hp[u][c] = params_at<BITS, GM, META>(rp, gsz, gshift, ur, c, K);
              }
          }
        }
      }
    };

    // Activation staging of step t: every thread stages E entries (all batch
    // rows of one 512-k step), issuing the same loads every step; halves past
    // K or past B read zeros (their offset lies outside the buffer
    // descriptor).  One wave instruction covers the 64 (unit, quad) entries of
    // one batch row, so its loads read that row's x contiguously; 4- and
    // 8-bit entries are eight consecutive k (one 16-byte load), 2- and 3-bit
    // entries two runs of four (two 8-byte loads).  In LDS, entry (m = unit
    // slot * Q + quad, batch tile, lane group h, batch row i16) sits at
    // (m * BT + bt) * 64 + 16 h + (i16 ^ (m & 15)): the swizzle spreads one
    // wave's scattered writes over all banks, and the MFMA operand reads stay
    // one contiguous block per 16 lanes.  Offsets are worked out once per
    // round; a step only advances them by the step's K extent.
    static_assert(UT * Q == 64, "one wave instruction stages one batch row of a step");
    int xk[E][2];           // first k of each half at step 0 (K: never valid)
    uint32_t xo[E][2];      // byte offset of that k in x
    int xl[E];              // LDS entry of the thread's entry
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int e = tid + i * kThreads;
      const int ml = e & 63, b = e >> 6;
      const int ul = ml / Q, q = ml % Q;      // unit of the step, quad
      // inverse of part_unit: K part, lane group and unit index of unit ul
      const int ekp = ul / (4 * NW), pr = ul % (4 * NW);
      const int run = pr / (4 * RN), pw = pr % (4 * RN);
      const int eh = pw / RN, eu = run * RN + pw % RN;
      const UnitRef ur = unit_at(0, ul);
      const int kl = unit_k<BITS>(ur, U::lo(4 * q)), kh = unit_k<BITS>(ur, U::hi(4 * q));
      xk[i][0] = b < B ? kl : K;
      xk[i][1] = b < B ? kh : K;
      xo[i][0] = 2u * ((uint32_t)b * (uint32_t)K + (uint32_t)kl);
      xo[i][1] = 2u * ((uint32_t)b * (uint32_t)K + (uint32_t)kh);
      const int m = (ekp * NW + eu) * Q + q;
      xl[i] = (m * BT + (b >> 4)) * 64 + 16 * eh + ((b & 15) ^ (m & 15));
    }
    uint4 xr[E];
    auto fetch_x = [&](int t) {
      const int tk = t * kTileK;
      const uint32_t tb = 2u * (uint32_t)tk;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const uint32_t ol = xk[i][0] + tk < K ? xo[i][0] + tb : 0xFFFFFFF0u;
        if constexpr (BITS == 4 || BITS == 8) {
          const u4_t v = __builtin_amdgcn_raw_buffer_load_b128(xrs, ol, 0, 0);
          xr[i] = make_uint4(v.x, v.y, v.z, v.w);
        } else {
          const uint32_t oh = xk[i][1] + tk < K ? xo[i][1] + tb : 0xFFFFFFF0u;
          const auto la = __builtin_amdgcn_raw_buffer_load_b64(xrs, ol, 0, 0);
          const auto lb = __builtin_amdgcn_raw_buffer_load_b64(xrs, oh, 0, 0);
          xr[i] = make_uint4(la[0], la[1], lb[0], lb[1]);
        }
      }
    };
    auto store_x = [&](int buf) {
      uint4* xs = lds + buf * XBUF;
#pragma unroll
      for (int i = 0; i < E; ++i)
        xs[xl[i]] = BITS == 8 ? xr[i]  // 8-bit slots pair neighbouring codes: x as loaded
                              : make_uint4(__builtin_amdgcn_perm(xr[i].z, xr[i].x, 0x05040100u),
                               __builtin_amdgcn_perm(xr[i].z, xr[i].x, 0x07060302u),
                               __builtin_amdgcn_perm(xr[i].w, xr[i].y, 0x05040100u),
                               __builtin_amdgcn_perm(xr[i].w, xr[i].y, 0x07060302u));
    };

    auto compute = [&](int t, int buf, WBuf& b) {
      if (!active) return;
      const uint4* xs = lds + buf * XBUF;
      // One MFMA takes, for each of the 16 rows, 32 codes from 4 units (one
      // per lane group) that lie in one span of 4 * RN consecutive units.
      // One group per row, or groups that hold every such span whole: the
      // codes enter as the exact integers q - z and the sum is scaled in fp32
      // afterwards (per unit for groups).  Other group layouts: the exact
      // dequantized value (q - z) * s enters as two fp16 operands, its fp16
      // rounding hi and the exact remainder lo, one MFMA each.
      // Staged step parameters of this lane's row (see kStepStage): group
      // i of the step belongs to run i.
      HalfParams shp[NVMAX];
      if constexpr (kStepStage) {
        {
          const uint32_t* d = ps + buf * 1024 + 8 * (16 * gl + i16);
          uint16_t sv[NVMAX];
          int32_t zv[NVMAX];
          uint32_t wv[NVMAX];
          if constexpr (NVMAX == 4) {
            const uint4 v = *reinterpret_cast<const uint4*>(d + 4);
            wv[0] = v.x, wv[1] = v.y, wv[2] = v.z, wv[3] = v.w;
          } else {
            const uint2 v = *reinterpret_cast<const uint2*>(d + 4);
            wv[0] = v.x, wv[1] = v.y;
          }
          if constexpr (META) {
#pragma unroll
            for (int i = 0; i < NVMAX; ++i) sv[i] = (uint16_t)wv[i], zv[i] = (int32_t)wv[i] >> 16;
          } else {
            uint32_t s2[2];
            if constexpr (NVMAX == 4) {
              const uint2 v = *reinterpret_cast<const uint2*>(d);
              s2[0] = v.x, s2[1] = v.y;
            } else {
              s2[0] = d[0], s2[1] = 0u;
            }
#pragma unroll
            for (int i = 0; i < NVMAX; ++i) {
              sv[i] = (uint16_t)(s2[i >> 1] >> (16 * (i & 1)));
              zv[i] = (int32_t)wv[i];
            }
          }
#pragma unroll
          for (int i = 0; i < NVMAX; ++i) shp[i] = HalfParams{sv[i], sv[i], zv[i], zv[i], true, true};
        }
      }
#pragma unroll
      for (int u = 0; u < NWMAX; ++u) {
        if (u < NW) {
          const UnitRef ur = my_unit(t, u);
          HalfParams hp[NC];
          PConsts<BITS> cc[NC];
          bool fast = true;
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            if constexpr (PERROW) {
              hp[c] = rowp;
              cc[c] = rowc;
              fast = rowfast;
            } else {
              if constexpr (kStepStage)
                hp[c] = shp[kRuns2 ? u >> 1 : u];
              else
                hp[c] = b.hp[GM == kWideGroups ? run_start(u) : u][c];
              fast &= make_pconsts<BITS>(hp[c], cc[c], DIRECT);
            }
            hp[c].v_lo = ur.va;
            hp[c].v_hi = ur.vb;
          }
          // entries of (kp, u) for this lane: [s][bt] blocks of 64, swizzled
          const int m0 = (kp * NW + u) * Q;
          const uint4* xe = xs + (m0 * BT) * 64 + h * 16;
          f4_t at[BT];  // wide groups: this unit's sums, scaled into acc below
          // fresh: the unit's first MFMA starts at[] from zero
          auto mma = [&](int s, const h2_t (&d)[4], bool fresh) {
            const h8_t bv = __builtin_bit_cast(
                h8_t, make_uint4(as_u32(d[0]), as_u32(d[1]), as_u32(d[2]), as_u32(d[3])));
#pragma unroll
            for (int bt = 0; bt < BT; ++bt) {
              const h8_t av =
                  __builtin_bit_cast(h8_t, xe[(s * BT + bt) * 64 + (i16 ^ ((m0 + s) & 15))]);
              if constexpr (GM == kWideGroups)
                at[bt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    av, bv, fresh ? f4_t{0.0f, 0.0f, 0.0f, 0.0f} : at[bt], 0, 0, 0);
              else
                acc[bt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc[bt], 0, 0, 0);
            }
          };
          if (__all(fast)) {
#pragma unroll
            for (int s = 0; s < Q; ++s) {
              h2_t qz[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int sl = 4 * s + e;
                qz[e] = qz_pair<BITS>(b.w[u], sl, mgp, cc[NC == 1 ? 0 : U::cset(sl)]);
              }
              if constexpr (DIRECT) {
                h2_t hi[4], lo[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const h2_t s2 = cc[NC == 1 ? 0 : U::cset(4 * s + e)].s2;
                  hi[e] = qz[e] * s2;
                  lo[e] = __builtin_elementwise_fma(qz[e], s2, -hi[e]);
                }
                mma(s, hi, false);
                mma(s, lo, false);
              } else {
                mma(s, qz, s == 0);
              }
            }
          } else {
            // exact per-code path (zero points far from the codes, or, for
            // the two-operand layouts, scales of 32 and more): the value --
            // q - z, or (q - z) * s -- formed in fp32 and entered as its fp16
            // rounding plus the remainder; one quad per loop trip, the unit's
            // words read back from this wave's LDS scratch
            uint32_t* wsc = slow_scratch + wave * (W * 64);
#pragma unroll
            for (int i = 0; i < W; ++i) wsc[i * 64 + lane] = b.w[u][i];
#pragma unroll
            for (int bt = 0; bt < BT; ++bt) at[bt] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 1
            for (int s = 0; s < Q; ++s) {
              h2_t hi[4], lo[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int sl = 4 * s + e;
                const HalfParams& hh = (NC == 1 || U::cset(sl) == 0) ? hp[0] : hp[NC - 1];
                float vl = (float)((int)unit_code_lds<BITS>(wsc, lane, U::lo(sl)) - hh.z_lo);
                float vh = (float)((int)unit_code_lds<BITS>(wsc, lane, U::hi(sl)) - hh.z_hi);
                if constexpr (DIRECT) {
                  vl *= h_bits_to_f32(hh.s_lo);
                  vh *= h_bits_to_f32(hh.s_hi);
                }
                uint16_t hl, ll, hh16, lh;
                split_f16(vl, hl, ll);
                split_f16(vh, hh16, lh);
                hi[e] = as_h2((uint32_t)hl | ((uint32_t)hh16 << 16));
                lo[e] = as_h2((uint32_t)ll | ((uint32_t)lh << 16));
              }
              mma(s, hi, false);
              mma(s, lo, false);
            }
          }
          if constexpr (GM == kWideGroups) {
            const float su = h_bits_to_f32(hp[0].s_lo);
#pragma unroll
            for (int bt = 0; bt < BT; ++bt) acc[bt] += su * at[bt];
          }
        }
      }
    };

    // One step per activation tile.  Step t: fetch x of step t+1, load the
    // weights of step t+1, multiply step t, store x of step t+1, barrier.  The
    // loads past the last step are clamped and their data unused; issuing
    // them anyway keeps every wait exact (the decode waits only for its own
    // weights, the store only for the activations).
    WBuf wa, wb;
    fetch_x(0);
    load_w(0, wa);
    if constexpr (kStepStage) fetch_p(0);
    store_x(0);
    if constexpr (kStepStage) store_p(0);
    __syncthreads();
    for (int t = 0; t < T; t += 2) {
      fetch_x(min(t + 1, T - 1));
      load_w(min(t + 1, T - 1), wb);
      if constexpr (kStepStage) fetch_p(min(t + 1, T - 1));
      compute(t, 0, wa);
      if (t + 1 < T) {
        store_x(1);
        if constexpr (kStepStage) store_p(1);
      }
      __syncthreads();
      if (t + 1 >= T) break;
      fetch_x(min(t + 2, T - 1));
      load_w(min(t + 2, T - 1), wa);
      if constexpr (kStepStage) fetch_p(min(t + 2, T - 1));
      compute(t + 1, 1, wb);
      if (t + 2 < T) {
        store_x(0);
        if constexpr (kStepStage) store_p(0);
      }
      __syncthreads();
    }

    // K parts meet in LDS: red[(gl * KP + kp)][b][j], b < BP, j < 16
    float* red = reinterpret_cast<float*>(lds);
    if (active) {
#pragma unroll
      for (int bt = 0; bt < BT; ++bt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int b = 16 * bt + 4 * h + r;
          red[((gl * KP + kp) * BP + b) * 16 + i16] = PERROW ? acc[bt][r] * row_scale : acc[bt][r];
        }
    }
    __syncthreads();
    const int outs = RG * 16 * B;
    for (int e = tid; e < outs; e += kThreads) {
      const int j = e & 15;
      const int rest = e >> 4;
      const int g = rest % RG, b = rest / RG;
      const int row = 16 * (gr0 + g) + j;
      float v = 0.0f;
      for (int p = 0; p < KP; ++p) v += red[((g * KP + p) * BP + b) * 16 + j];
      if (row < N) y[(int64_t)b * N + row] = f32_to_h_bits(v);
    }
    __syncthreads();  // the LDS is reused by the next round
  }
}

// Every round of every workgroup takes at least five 16-row groups (one K
// part per round): workgroups own ng or ng + 1 groups, walked in rounds of
// eight.
inline bool rounds_one_part(int N) {
  const int NG = (N + 15) / 16;
  const int cus = device_cu_count();
  const int nwg = NG < cus ? NG : cus;
  const int gb = NG / nwg, ge = NG % nwg;
  auto ok = [](int ng) { return ng >= 5 && (ng % kWaves == 0 || ng % kWaves >= 5); };
  return (nwg == ge || ok(gb)) && (ge == 0 || ok(gb + 1));
}

template <int BITS, int BT, int GM, bool META, bool SS = false>
hipError_t launch_t(const uint16_t* x, int B, const uint32_t* packed, const uint16_t* scales,
                    const int32_t* zeros, int N, int K, int G, int gsz, int gshift, uint16_t* y,
                    hipStream_t stream) {
  size_t lds = 2 * (size_t)kTileK * 16 * BT * 2 + (size_t)kWaves * Unit<BITS>::WORDS * 64 * 4;
  if (lds > device_lds_per_block()) return hipErrorNotSupported;
  // wide groups whose group is exactly one step's run span: stage each
  // wave's scales and zeros in LDS when they fit (the kernel's layout:
  // strides G/2 + 2 and G + 4 words per row, 16 rows per wave)
  int pstage = 0;
  if constexpr (GM == kWideGroups && BT == 4) {
    // 64-row batch tiles: the variant that stages each step's parameters
    // (8 KB, see the kernel) when the group is exactly one run's span, K is
    // whole steps, the arrays are 16-byte aligned and every round has one K
    // part
    const size_t extra = 2 * 1024 * 4;
    if constexpr (SS) {
      lds += extra;
    } else {
      const int span = 4 * (BITS == 8 ? 2 : 1) * Unit<BITS>::CODES;
      const bool aligned = reinterpret_cast<uintptr_t>(scales) % 16 == 0 &&
                           (META || reinterpret_cast<uintptr_t>(zeros) % 16 == 0);
      // (byte offsets into the parameter arrays are 32-bit)
      if (gsz == span && K % kTileK == 0 && aligned && rounds_one_part(N) &&
          (int64_t)N * G * 4 <= 0x7fffffff && lds + extra <= device_lds_per_block())
        return launch_t<BITS, BT, GM, META, true>(x, B, packed, scales, zeros, N, K, G, gsz,
                                                  gshift, y, stream);
    }
  }
  if (GM == kWideGroups && BT <= 2) {
    const int span = 4 * (BITS == 8 ? 2 : 1) * Unit<BITS>::CODES;
    const size_t pww = META ? 16 * (size_t)(G + 4) : 16 * (size_t)(G / 2 + 2 + G + 4);
    const size_t extra = (size_t)kWaves * pww * 4;
    const bool aligned = reinterpret_cast<uintptr_t>(scales) % 16 == 0 &&
                         (META || reinterpret_cast<uintptr_t>(zeros) % 16 == 0);
    if (gsz == span && G % 8 == 0 && aligned && lds + extra <= device_lds_per_block()) {
      pstage = 1;
      lds += extra;
    }
  }
  const auto kern = qgemm_kernel<BITS, BT, GM, META, SS>;
  // the LDS request exceeds the default limit: raise it, once per device, to
  // the most any launch of this kernel can ask for
  const hipError_t e =
      raise_lds_limit(reinterpret_cast<const void*>(kern), (int)device_lds_per_block());
  if (e != hipSuccess) return e;
  const int NG = (N + 15) / 16;
  const int cus = device_cu_count();
  const int grid = NG < cus ? NG : cus;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds, stream, x, B, packed, scales, zeros,
                     y, N, K, G, gsz, gshift, pstage);
  return hipGetLastError();
}

template <int BITS, int GM, bool META>
hipError_t launch_bits(int B, const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                       const int32_t* zeros, int N, int K, int G, int gsz, int gshift,
                       uint16_t* y, hipStream_t stream) {
  // batches beyond 64 rows run as several passes over the weights
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int bc = B - b0 < 64 ? B - b0 : 64;
    const uint16_t* xb = x + (int64_t)b0 * K;
    uint16_t* yb = y + (int64_t)b0 * N;
    hipError_t e;
    if (bc <= 16)
      e = launch_t<BITS, 1, GM, META>(xb, bc, packed, scales, zeros, N, K, G, gsz, gshift, yb,
                                      stream);
    else if (bc <= 32)
      e = launch_t<BITS, 2, GM, META>(xb, bc, packed, scales, zeros, N, K, G, gsz, gshift, yb,
                                      stream);
    else
      e = launch_t<BITS, 4, GM, META>(xb, bc, packed, scales, zeros, N, K, G, gsz, gshift, yb,
                                      stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Group layout dispatch of one width (wide groups do not apply to 3-bit).
template <int BITS, bool META>
hipError_t launch_layout(int gm, int B, const uint16_t* x, const uint32_t* packed,
                         const uint16_t* scales, const int32_t* zeros, int N, int K, int G,
                         int gsz, int gshift, uint16_t* y, hipStream_t stream) {
  switch (gm) {
    case kPerRow:
      return launch_bits<BITS, kPerRow, META>(B, x, packed, scales, zeros, N, K, G, gsz, gshift,
                                              y, stream);
    case kPow2Groups:
      return launch_bits<BITS, kPow2Groups, META>(B, x, packed, scales, zeros, N, K, G, gsz,
                                                  gshift, y, stream);
    case kWideGroups:
      return launch_bits<BITS, (BITS == 3 ? kPow2Groups : kWideGroups), META>(
          B, x, packed, scales, zeros, N, K, G, gsz, gshift, y, stream);
    default:
      return launch_bits<BITS, kAnyGroups, META>(B, x, packed, scales, zeros, N, K, G, gsz,
                                                 gshift, y, stream);
  }
}

template <bool META>
hipError_t launch_width(int bits, int gm, int B, const uint16_t* x, const uint32_t* packed,
                        const uint16_t* scales, const int32_t* zeros, int N, int K, int G,
                        int gsz, int gshift, uint16_t* y, hipStream_t stream) {
  switch (bits) {
    case 2:
      return launch_layout<2, META>(gm, B, x, packed, scales, zeros, N, K, G, gsz, gshift, y,
                                    stream);
    case 3:
      return launch_layout<3, META>(gm, B, x, packed, scales, zeros, N, K, G, gsz, gshift, y,
                                    stream);
    case 8:
      return launch_layout<8, META>(gm, B, x, packed, scales, zeros, N, K, G, gsz, gshift, y,
                                    stream);
    default:
      return launch_layout<4, META>(gm, B, x, packed, scales, zeros, N, K, G, gsz, gshift, y,
                                    stream);
  }
}

}  // namespace

hipError_t launch_qgemm(const uint16_t* x, int64_t B, const uint32_t* packed,
                        const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K,
                        int bits, int64_t group_size, bool meta, uint16_t* y,
                        hipStream_t stream) {
  const int gsz = (int)(group_size == 0 ? K : group_size);
  const int G = (int)(K / gsz);
  const int gshift = (gsz & (gsz - 1)) == 0 ? __builtin_ctz((unsigned)gsz) : -1;
  // wide groups: every MFMA's span of units (4 x 32 codes at 4 bits, 4 x 64
  // at 2 bits, 8 x 16 at 8 bits, starting on a multiple of the span) lies in
  // one group
  const bool wide = bits != 3 && gshift >= 0 && gsz >= (bits == 2 ? 256 : 128);
  const int gm = G == 1 ? kPerRow : wide ? kWideGroups : gshift >= 0 ? kPow2Groups : kAnyGroups;
  const int b = (int)B, n = (int)N, k = (int)K;
  return meta ? launch_width<true>(bits, gm, b, x, packed, scales, zeros, n, k, G, gsz, gshift, y,
                                   stream)
              : launch_width<false>(bits, gm, b, x, packed, scales, zeros, n, k, G, gsz, gshift,
                                    y, stream);
}

}  // namespace lowbit
