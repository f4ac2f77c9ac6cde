// gemv_mma.hip -- dequantize + small-batch product (1..16 activation rows) on
// the fp16 matrix cores, for 2- and 4-bit codes whose groups hold whole
// 16-byte units (2-bit: groups of a multiple of 64 codes; 4-bit: of 32).
//
// y[m][n] = sum_k x[m][k] * (q[n][k] - z) * s, the exact value of each code
// on the min-max RTN grid (BladeLLM model quantization, "Quantization
// algorithms", MinMax; groups along input channels: "block_wise_quant"),
// decoded by the GPU's own cores inside the product ([Feature Request] 4bit
// and 2bit and 1bit quantization support).  Per group,
//     sum_{k in g} x_k (q_k - z) s = s * (sum_{k in g} x_k q_k - z * S_g),
//     S_g = sum_{k in g} x_k,
// so the decode produces the exact fp16 integer q (one bitwise OR into the
// exponent pattern of 2^(10 - p), one packed subtraction of 2^(10 - p): the
// same constants for every group), the matrix cores sum x * q in fp32, and
// the zero point enters once per group in fp32 through the activation sums
// S_g, which depend on x alone and are formed while x is staged.  Nothing
// depends on the zero point's size, so no exact slow path is needed.
//
// Layout on gfx950 (one workgroup of 16 waves per CU, or two of 8 waves up to
// 8 activation rows):
//  - the weight rows form tiles of 16 (the MFMA's 16 columns n); a K step of
//    a tile is 4 consecutive 16-byte units of each row: lane (n, h) loads
//    unit h of its row (the row's four lanes read 64 contiguous bytes), then
//    a 4 x 4 word transpose across the four lanes (two v_permlane32_swap and
//    two v_permlane16_swap) leaves lane (n, h) with word h of each of the 4
//    units, so every MFMA column covers codes of one unit, hence one group;
//  - lane (n, h) also loads the scale and zero point of unit h of its row
//    (one small load each), and three lane swaps give every lane of row n
//    those of all four units;
//  - the activations of the B batch rows are staged in LDS in rounds of K,
//    already in the operand order of the matrix cores, together with the
//    per-unit sums S; lanes of operand rows m >= B read row B - 1, which
//    only reaches output rows that are never stored;
//  - every wave takes the same share of (tile, K step) pairs in every round
//    and keeps one fp32 accumulator per tile it touches across the rounds;
//    the next round's activations and weights are requested before the
//    current round is multiplied; at the end the waves' partial sums meet in
//    LDS and are added in a fixed order (deterministic).
#include "common.h"
#include "kernels.h"
#include "unit_decode.h"

namespace lowbit {

namespace {

// Workgroups of W waves, 16 / W of them per CU: one of 16 waves, or two of
// 8 (each then stages its own rounds, so one computes while the other waits
// for its weights; measured faster up to 8 activation rows)
template <int W>
constexpr int kWgPerCu = 16 / W;
// K steps per wave and round: two (three would not fit the 128 registers of a
// 16-wave workgroup with separate scale and zero arrays; the compact-word
// variant takes the same share so that both sum in the same order)
constexpr int kAMax = 2;
// LDS for one round of activations: 64 KB with one workgroup per CU, 56 KB
// with two
template <int W>
constexpr size_t kXsBudget = W == 16 ? 64 * 1024 : 56 * 1024;
constexpr size_t kLdsCap = 160 * 1024;      // gfx950 LDS per CU
// an LDS request that leaves room for kWgPerCu workgroups per CU and no more
template <int W>
constexpr size_t kWgLds = kLdsCap / (kWgPerCu<W> + 1) + 1024;

typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

// Geometry of a 16-byte unit.  2-bit: 64 codes, word h holds codes 16h..16h+15
// as 8 pairs (c, c + 8); one unit feeds two MFMAs (pairs 0..3, 4..7).  4-bit:
// 32 codes, word h holds codes 8h..8h+7 as 4 pairs (c, c + 4); one MFMA.
template <int BITS>
struct MU;
template <>
struct MU<2> {
  static constexpr int CODES = 64, SUBS = 2, WCODES = 16, PAIRS = 8, HALF = 8;
};
template <>
struct MU<4> {
  static constexpr int CODES = 32, SUBS = 1, WCODES = 8, PAIRS = 4, HALF = 4;
};

// The exact fp16 integers (q_c, q_{c + HALF}) of pair c of a word: the field
// sits at bit p of both halves (after a shift for the upper pairs), OR-ed
// into the pattern of 2^(10 - p) it is 2^(10 - p) + q, and subtracting the
// same pattern leaves q.  mg[i] holds the pattern for p = i * BITS.
template <int BITS>
__device__ __forceinline__ h2_t q_pair(uint32_t w, uint32_t wsh, int c, const uint32_t (&mg)[5]) {
  if constexpr (BITS == 2) {
    const bool up = c >= 5;
    const int p = up ? 2 * (c - 5) : 2 * c;
    const uint32_t v = up ? wsh : w;
    return as_h2((v & (0x00030003u << p)) | mg[p >> 1]) - as_h2(mg[p >> 1]);
  } else {
    const bool up = c >= 2;
    const int p = up ? 4 * (c - 2) : 4 * c;
    const uint32_t v = up ? wsh : w;
    return as_h2((v & (0x000F000Fu << p)) | mg[p >> 2]) - as_h2(mg[p >> 2]);
  }
}

// n / d for n < 2^16 and 1 <= d <= 2^16 as the high half of n * ceil(2^32 / d)
// (the rounding-up error, below d / 2^32 per unit of n, stays under 1 / d);
// d = 1 is passed as 0.
inline uint32_t small_recip(int d) {
  return d == 1 ? 0u : (uint32_t)((((uint64_t)1 << 32) + (uint64_t)d - 1) / (uint64_t)d);
}
__device__ __forceinline__ uint32_t small_quotient(uint32_t n, uint32_t recip) {
  return recip ? __umulhi(n, recip) : n;
}

template <int BITS, bool META, int A, int W>
__global__ __launch_bounds__(W * 64, kWgPerCu<W>) void qgemv_mma_kernel(
    const uint16_t* __restrict__ x, int B, const uint32_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros,
    uint16_t* __restrict__ y, int N, int K, int G, uint32_t upg_recip, uint32_t b_recip, int RK,
    int nrounds) {
  using M = MU<BITS>;
  constexpr int U = M::CODES, SUBS = M::SUBS, TPU = U / 32;
  extern __shared__ uint4 lds[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 15, h = lane >> 4;
  const uint32_t row_bytes = (uint32_t)K * BITS / 8;
  const int row_words = (int)(row_bytes / 4);
  const int units_per_row = K / U;
  const int SR = RK / 4;  // K steps per round and tile

  // this workgroup's tiles
  const int NT = (N + 15) / 16;
  const int nwg = (int)gridDim.x, wg = (int)blockIdx.x;
  const int tb = NT / nwg, tx = NT % nwg;
  const int t0 = wg * tb + min(wg, tx);
  const int ntiles = tb + (wg < tx ? 1 : 0);

  // LDS: activation entries [RK][SUBS][4 h][B m] (16 B each), sums S
  // [RK][16 m] (fp32), partial sums [wave][A][16 n][16 m] (fp32).  Rows
  // m >= B of the matrix-core operand and of S are never written: they only
  // reach rows m >= B of the products, which are never stored.
  const int xentries = RK * SUBS * 4 * B;
  uint4* xs = lds;
  float* ssum = reinterpret_cast<float*>(xs + xentries);
  float* part = ssum + RK * 16;

  // this wave's (tile, step) pairs: the same indices every round
  const int total = ntiles * SR;
  const int a = (total + W - 1) / W;  // <= A (host)
  const int i0 = wave * a;
  const int tile_first = i0 / SR;

  uint32_t mg[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int p = i * BITS;
    uint32_t v = p <= 10 ? (uint32_t)(25 - p) * 0x04000400u : 0u;
    asm volatile("" : "+v"(v));  // keep each pattern in its own vector register
    mg[i] = v;
  }

  // A step's words and the group parameters of the lane's own unit (lane
  // (n, h) holds unit h of its row): the compact word (META), or the scale
  // bits and the zero point.
  struct Step {
    uint32_t w[4];
    uint32_t p;
    int32_t z;
  };
  // Loads of the wave's step i of round r (an empty range past the share or
  // past N: zeros, no memory traffic).
  // One descriptor per load instruction, wave-uniform: the tile's rows that
  // exist (rows past N read zeros), each lane at its row's offset.  A unit
  // past a row's end (the last step of a round) reads the next row's bytes;
  // those codes meet zero activations and zero sums, so they add exactly 0.
  auto load_step = [&](int r, int i, Step& st) __attribute__((always_inline)) {
    const int idx = i0 + i;
    const bool valid = i < a && idx < total;
    const int tl = valid ? idx / SR : 0;
    const int gs = r * SR + (valid ? idx - tl * SR : 0);  // the row's K step
    const int row0 = (t0 + tl) * 16;
    const int rc = min(row0 + nl, N - 1);
    const uint32_t bytes = valid ? (uint32_t)min(16, N - row0) * row_bytes : 0u;
    const uint64_t base = reinterpret_cast<uint64_t>(packed + (int64_t)row0 * row_words);
    const uint32_t blo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base);
    const uint32_t bhi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32));
    const uint32_t sz = (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(((uint64_t)bhi << 32) | blo), (short)0, (int)sz, 0x00020000);
    const u4_t v = __builtin_amdgcn_raw_buffer_load_b128(
        rs, (uint32_t)nl * row_bytes + (uint32_t)(4 * gs + h) * 16u, 0, 2);
    st.w[0] = v.x, st.w[1] = v.y, st.w[2] = v.z, st.w[3] = v.w;
    // group of unit 4 gs + h
    const uint32_t uh = (uint32_t)(4 * gs + h);
    const uint32_t gu = small_quotient(uh, upg_recip);
    const int64_t g = (int64_t)rc * G + min((int)gu, G - 1);
    if constexpr (META) {
      st.p = reinterpret_cast<const uint32_t*>(scales)[g];
      st.z = 0;
    } else {
      st.p = scales[g];
      st.z = zeros[g];
    }
  };

  // Round r's activations: TPU threads per (unit, batch row) pair, each
  // staging 32 codes (2-bit: hh 0..1 or 2..3; 4-bit: the whole unit); pair
  // e / TPU is unit e / (TPU B) of the round for batch row (e / TPU) % B
  // (zeros past the row's units).  The loads are issued apart from the
  // stores so that they can overlap other loads.
  struct XR {
    uint4 c[4];
  };
  auto stage_load = [&](int r, XR& xr) __attribute__((always_inline)) {
    const int q = tid / TPU, half = tid - q * TPU;
    const int ur = (int)small_quotient((uint32_t)q, b_recip), m = q - ur * B;
    const int ug = r * RK + ur;
    const bool v = q < RK * B && ug < units_per_row;
    const uint4* xp = reinterpret_cast<const uint4*>(x + (int64_t)m * K +
                                                     (int64_t)(v ? ug : 0) * U + 32 * half);
#pragma unroll
    for (int c = 0; c < 4; ++c) xr.c[c] = xp[c];
  };
  auto stage_store = [&](int r, const XR& xr) __attribute__((always_inline)) {
    // the store addresses are formed here, not kept live across the rounds
    int te = tid;
    asm volatile("" : "+v"(te));
    const int q = te / TPU, half = te - q * TPU;
    const int ur = (int)small_quotient((uint32_t)q, b_recip), m = q - ur * B;
    const bool v = r * RK + ur < units_per_row;
    float sum = 0.0f;
    if (q < RK * B) {
#pragma unroll
      for (int hl = 0; hl < 4 / TPU; ++hl) {
        const int hh = hl + half * (4 / TPU);
#pragma unroll
        for (int sub = 0; sub < SUBS; ++sub) {
          // codes k0 .. k0+3 and k0+HALF .. k0+HALF+3 of the unit (k0 local
          // to the thread's 32 codes)
          const int k0 = hl * M::WCODES + 4 * sub;
          const uint4 cl = xr.c[k0 / 8], ch = xr.c[(k0 + M::HALF) / 8];
          uint2 l = (k0 % 8) ? make_uint2(cl.z, cl.w) : make_uint2(cl.x, cl.y);
          uint2 g = ((k0 + M::HALF) % 8) ? make_uint2(ch.z, ch.w) : make_uint2(ch.x, ch.y);
          if (!v) l = make_uint2(0u, 0u), g = make_uint2(0u, 0u);
          const h2_t l0 = as_h2(l.x), l1 = as_h2(l.y), g0 = as_h2(g.x), g1 = as_h2(g.y);
          sum += ((float)l0.x + (float)l0.y) + ((float)l1.x + (float)l1.y) +
                 ((float)g0.x + (float)g0.y) + ((float)g1.x + (float)g1.y);
          xs[((ur * SUBS + sub) * 4 + hh) * B + m] =
              make_uint4(__builtin_amdgcn_perm(g.x, l.x, 0x05040100u),
                         __builtin_amdgcn_perm(g.x, l.x, 0x07060302u),
                         __builtin_amdgcn_perm(g.y, l.y, 0x05040100u),
                         __builtin_amdgcn_perm(g.y, l.y, 0x07060302u));
        }
      }
    }
    // the two halves of a 2-bit unit sit in neighbouring lanes
    if constexpr (TPU == 2) sum += __shfl_xor(sum, 1, kWave);
    if (q < RK * B && half == 0) ssum[ur * 16 + m] = sum;
  };

  f4_t acc[A];
#pragma unroll
  for (int j = 0; j < A; ++j) acc[j] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int mrow = min(nl, B - 1);  // operand row read by lane (n, h)

  // The wave's steps of round r: transpose, decode, multiply, group epilogue.
  auto compute = [&](int r, Step (&st)[A]) __attribute__((always_inline)) {
    // the lane's operand entry, formed here so that the compiler keeps one
    // address per round rather than one per unit live across the rounds
    int xl = h * B + mrow, sl = 4 * h;
    asm volatile("" : "+v"(xl), "+v"(sl));
    const uint4* xsl = xs + xl;
    const float* ssl = ssum + sl;
#pragma unroll
    for (int i = 0; i < A; ++i) {
      const int idx = i0 + i;
      if (!(i < a && idx < total)) continue;  // wave-uniform
      const int tl = idx / SR;
      const int sr = idx - tl * SR;
      const int seg = tl - tile_first;
      // word h of each unit in lane (n, h): a 4 x 4 transpose across the
      // row's four lanes (16 apart)
      uint32_t w0 = st[i].w[0], w1 = st[i].w[1], w2 = st[i].w[2], w3 = st[i].w[3];
      {
        auto p02 = __builtin_amdgcn_permlane32_swap(w0, w2, false, false);
        auto p13 = __builtin_amdgcn_permlane32_swap(w1, w3, false, false);
        auto q01 = __builtin_amdgcn_permlane16_swap(p02[0], p13[0], false, false);
        auto q23 = __builtin_amdgcn_permlane16_swap(p02[1], p13[1], false, false);
        w0 = q01[0], w1 = q01[1], w2 = q23[0], w3 = q23[1];
      }
      // the parameters of unit u, held by lane (n, u), in every lane of row n
      uint32_t pu[4];
      int32_t zu[4];
      {
        auto p = __builtin_amdgcn_permlane32_swap(st[i].p, st[i].p, false, false);
        auto pa = __builtin_amdgcn_permlane16_swap(p[0], p[0], false, false);
        auto pb = __builtin_amdgcn_permlane16_swap(p[1], p[1], false, false);
        pu[0] = pa[0], pu[1] = pa[1], pu[2] = pb[0], pu[3] = pb[1];
        if constexpr (!META) {
          auto z = __builtin_amdgcn_permlane32_swap(st[i].z, st[i].z, false, false);
          auto za = __builtin_amdgcn_permlane16_swap(z[0], z[0], false, false);
          auto zb = __builtin_amdgcn_permlane16_swap(z[1], z[1], false, false);
          zu[0] = (int32_t)za[0], zu[1] = (int32_t)za[1], zu[2] = (int32_t)zb[0],
          zu[3] = (int32_t)zb[1];
        }
      }
      const uint32_t wt[4] = {w0, w1, w2, w3};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int ur = 4 * sr + u;  // unit within the round
        const uint32_t wsh = wt[u] >> (BITS == 2 ? 10 : 8);
        f4_t d = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int sub = 0; sub < SUBS; ++sub) {
          const h8_t bv = __builtin_bit_cast(
              h8_t, make_uint4(as_u32(q_pair<BITS>(wt[u], wsh, 4 * sub + 0, mg)),
                               as_u32(q_pair<BITS>(wt[u], wsh, 4 * sub + 1, mg)),
                               as_u32(q_pair<BITS>(wt[u], wsh, 4 * sub + 2, mg)),
                               as_u32(q_pair<BITS>(wt[u], wsh, 4 * sub + 3, mg))));
          const h8_t av = __builtin_bit_cast(h8_t, xsl[(ur * SUBS + sub) * 4 * B]);
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, d, 0, 0, 0);
        }
        // s * (sum x q - z * S) for the lane's four batch rows 4h .. 4h+3
        const float s = h_bits_to_f32((uint16_t)pu[u]);
        const int32_t zp = META ? (int32_t)pu[u] >> 16 : zu[u];
        const float sz = s * (float)zp;
        const f4_t sv = *reinterpret_cast<const f4_t*>(ssl + ur * 16);
#pragma unroll
        for (int j = 0; j < A; ++j) {
          if (j != seg) continue;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[j][e] = __builtin_fmaf(s, d[e], acc[j][e]);
            acc[j][e] = __builtin_fmaf(-sz, sv[e], acc[j][e]);
          }
        }
      }
    }
  };

  // Round r + 1's activations and weights are requested before round r is
  // multiplied (the last round requests nothing); the activation loads go
  // first, so that waiting for them does not wait for the weights.
  XR xr;
  Step sa[A], sb[A];
  stage_load(0, xr);
#pragma unroll
  for (int i = 0; i < A; ++i) load_step(0, i, sa[i]);
  stage_store(0, xr);
  __syncthreads();
  for (int r = 0;; r += 2) {
    if (r + 1 >= nrounds) {
      compute(r, sa);
      break;
    }
    stage_load(r + 1, xr);
#pragma unroll
    for (int i = 0; i < A; ++i) load_step(r + 1, i, sb[i]);
    compute(r, sa);
    __syncthreads();
    stage_store(r + 1, xr);
    __syncthreads();
    if (r + 2 >= nrounds) {
      compute(r + 1, sb);
      break;
    }
    stage_load(r + 2, xr);
#pragma unroll
    for (int i = 0; i < A; ++i) load_step(r + 2, i, sa[i]);
    compute(r + 1, sb);
    __syncthreads();
    stage_store(r + 2, xr);
    __syncthreads();
  }

  // partial sums: lane (n, h) holds D[4h + e][n] of each tile segment
#pragma unroll
  for (int j = 0; j < A; ++j)
    *reinterpret_cast<f4_t*>(part + ((wave * A + j) * 16 + nl) * 16 + 4 * h) = acc[j];
  __syncthreads();
  // each output: the segments of its tile, in wave order
  for (int e = tid; e < ntiles * 16 * B; e += (W * kWave)) {
    const int tl = e / (16 * B);
    const int rest = e - tl * 16 * B;
    const int m = rest / 16, n = rest - m * 16;
    const int row = (t0 + tl) * 16 + n;
    float v = 0.0f;
    for (int w = 0; w < W; ++w) {
      const int wi0 = w * a;
      if (wi0 >= total) break;
      const int first = wi0 / SR;
      const int last = (min(wi0 + a, total) - 1) / SR;
      if (tl < first || tl > last) continue;
      v += part[((w * A + (tl - first)) * 16 + n) * 16 + m];
    }
    if (row < N) y[(int64_t)m * N + row] = f32_to_h_bits(v);
  }
}

template <int BITS, bool META, int A, int W>
hipError_t launch_mma_t(const uint16_t* x, int B, const uint32_t* packed,
                        const uint16_t* scales, const int32_t* zeros, int N, int K, int G,
                        uint32_t upg_recip, uint32_t b_recip, int RK, int nrounds, int nwg,
                        size_t lds, uint16_t* y, hipStream_t stream) {
  const auto kern = qgemv_mma_kernel<BITS, META, A, W>;
  const hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(kern),
                                       (int)(device_lds_per_block() < kLdsCap
                                                 ? device_lds_per_block()
                                                 : kLdsCap));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(W * kWave), lds, stream, x, B, packed, scales, zeros,
                     y, N, K, G, upg_recip, b_recip, RK, nrounds);
  return hipGetLastError();
}

template <int BITS, bool META, int W>
hipError_t launch_mma_w(const uint16_t* x, int B, const uint32_t* packed,
                           const uint16_t* scales, const int32_t* zeros, int N, int K, int G,
                           int gsz, uint16_t* y, hipStream_t stream) {
  constexpr int U = MU<BITS>::CODES;
  if (gsz % U != 0) return hipErrorNotSupported;
  const int upg = gsz / U;
  const int units_per_row = K / U;
  // group quotients by multiply-high (exact below 2^16 units)
  if (units_per_row + 4 > 65536 || upg > 65536) return hipErrorNotSupported;
  const uint32_t upg_recip = small_recip(upg), b_recip = small_recip(B);
  // activations are staged in 16-byte loads
  if (reinterpret_cast<uintptr_t>(x) % 16 != 0) return hipErrorNotSupported;
  const int NT = (N + 15) / 16;
  const int cus = device_cu_count();
  const int nwg = NT < kWgPerCu<W> * cus ? NT : kWgPerCu<W> * cus;
  const int tiles_per_wg = (NT + nwg - 1) / nwg;
  // units per round: all of the row if it fits, bounded by the activation
  // budget, by one staging pass of the workgroup, and by kAMax steps per wave
  int RK = (units_per_row + 3) / 4 * 4;
  const int by_lds = (int)(kXsBudget<W> / ((size_t)U * B * 2)) / 4 * 4;
  const int by_threads = W * kWave / (B * (U / 32)) / 4 * 4;
  const int by_steps = W * kAMax / tiles_per_wg * 4;
  RK = RK < by_lds ? RK : by_lds;
  RK = RK < by_threads ? RK : by_threads;
  RK = RK < by_steps ? RK : by_steps;
  if (RK < 4) return hipErrorNotSupported;
  // With several rounds, a round's (tile, step) pairs are dealt to the waves
  // in equal shares of a = ceil(pairs / W): prefer the longest round whose
  // pairs fill every wave's share (e.g. 8 steps rather than 10 over 8 waves,
  // where 10 would leave three waves idle).
  if (RK < units_per_row) {
    for (int rk = RK; rk >= 4; rk -= 4) {
      if ((tiles_per_wg * (rk / 4)) % W == 0) {
        RK = rk;
        break;
      }
    }
  }
  const int nrounds = (units_per_row + RK - 1) / RK;
  // K steps per wave and round in the workgroups with the most tiles
  const int steps = (tiles_per_wg * (RK / 4) + W - 1) / W;
  size_t lds = (size_t)RK * U * B * 2 + (size_t)RK * 16 * 4 + (size_t)W * steps * 256 * 4;
  if (lds > device_lds_per_block() || lds > kLdsCap / kWgPerCu<W>) return hipErrorNotSupported;
  if (lds < kWgLds<W> && kWgLds<W> <= device_lds_per_block()) lds = kWgLds<W>;
  switch (steps) {
    case 1:
      return launch_mma_t<BITS, META, 1, W>(x, B, packed, scales, zeros, N, K, G, upg_recip, b_recip,
                                         RK, nrounds, nwg, lds, y, stream);
    case 2:
      return launch_mma_t<BITS, META, 2, W>(x, B, packed, scales, zeros, N, K, G, upg_recip, b_recip,
                                         RK, nrounds, nwg, lds, y, stream);
    default:
      return hipErrorNotSupported;
  }
}

// Up to 8 activation rows: two 8-wave workgroups per CU; above: one of 16.
template <int BITS, bool META>
hipError_t launch_mma_bits(const uint16_t* x, int B, const uint32_t* packed,
                           const uint16_t* scales, const int32_t* zeros, int N, int K, int G,
                           int gsz, uint16_t* y, hipStream_t stream) {
  return B <= 8 ? launch_mma_w<BITS, META, 8>(x, B, packed, scales, zeros, N, K, G, gsz, y, stream)
                : launch_mma_w<BITS, META, 16>(x, B, packed, scales, zeros, N, K, G, gsz, y, stream);
}

}  // namespace

hipError_t launch_qgemv_mma(const uint16_t* x, int64_t B, const uint32_t* packed,
                            const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K,
                            int bits, int64_t group_size, bool meta, uint16_t* y,
                            hipStream_t stream) {
  if (B < 1 || B > 16 || group_size == 0) return hipErrorNotSupported;
  const int gsz = (int)group_size;
  const int G = (int)(K / gsz);
  const int b = (int)B, n = (int)N, k = (int)K;
  switch (bits) {
    case 2:
      return meta ? launch_mma_bits<2, true>(x, b, packed, scales, zeros, n, k, G, gsz, y, stream)
                  : launch_mma_bits<2, false>(x, b, packed, scales, zeros, n, k, G, gsz, y,
                                              stream);
    case 4:
      return meta ? launch_mma_bits<4, true>(x, b, packed, scales, zeros, n, k, G, gsz, y, stream)
                  : launch_mma_bits<4, false>(x, b, packed, scales, zeros, n, k, G, gsz, y,
                                              stream);
    default:
      return hipErrorNotSupported;
  }
}

}  // namespace lowbit
