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
// Layout of the work: a lane owns "chunks" of 8 consecutive weights (16 bytes
// of fp16, one 128-bit load).  Chunk c of a row is handled by thread c mod T
// of the row's workgroup, so every load and store instruction of a wave
// covers one contiguous span.  A chunk's 8 codes pack into 32 bits (4-bit),
// 16 bits (2-bit) or 24 bits (3-bit; four neighbouring lanes then assemble
// the three 32-bit words of their 32 codes with a DPP lane exchange).  The
// whole row stays in registers between the min/max pass and the code pass, so
// every weight is read from memory once.  At 8 bits a chunk's codes are its 8
// bytes in the packed row as well as in the byte-code output.
//
// Arithmetic.  The codes need fl32(w / s) exactly (one IEEE division per
// weight).  With r_hi = fl32(1/s) and r_lo = fl32(fma(-s, r_hi, 1) * r_hi),
// r_hi + r_lo equals 1/s to about 2^-47 relative, and
//     fl32(w / s) == fma(w, r_hi, fl32(w * r_lo))
// for every pair of fp16 values w and s > 0: the quotient of two 11-bit
// significands is never within 2^-36 (relative) of an fp32 rounding midpoint,
// while the right-hand side is within 2^-45 of w / s before its single
// rounding.  The identity was checked exhaustively over all fp16 w and all
// positive finite fp16 s, and for d / M (fp32 d, M = 3, 7, 15, 127, 255) over
// every fp32 significand.  Rounding to an integer uses v + 1.5 * 2^23, whose fp32 sum
// rounds v half-to-even onto the integer grid; the codes' quotients are
// bounded by 2^16 in magnitude (the largest |w| / s of any group of finite
// fp16 values), far inside the 2^22 range where that is exact.
#include "common.h"
#include "kernels.h"

#pragma clang fp contract(off)

namespace lowbit {

namespace {

typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

constexpr int kBufferDword3 = 0x00020000;      // raw 32-bit buffer format (gfx9 family)
constexpr int kSlc = 2;                        // weights are streamed: read once
constexpr float kRoundMagic = 12582912.0f;     // 1.5 * 2^23
constexpr uint32_t kRoundBits = 0x4B400000u;   // its bit pattern
constexpr uint32_t kPosInfPair = 0x7C007C00u;  // (+inf, +inf) as two fp16

// How a row's groups are reduced.
enum GroupMode {
  kRowGroup = 0,    // one group per row: wave reductions, one barrier
  kLaneGroups = 1,  // power-of-two groups of 4..64 chunks: lane butterflies, no LDS
  kLdsGroups = 2,   // any other group size: chunk extrema through LDS, a wave per group
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferDword3);
}

__device__ __forceinline__ uint32_t pk_min(uint32_t a, uint32_t b) {
  return as_u32(__builtin_elementwise_min(as_h2(a), as_h2(b)));
}
__device__ __forceinline__ uint32_t pk_max(uint32_t a, uint32_t b) {
  return as_u32(__builtin_elementwise_max(as_h2(a), as_h2(b)));
}
// The same on raw loaded weights.  The builtins above first quiet possible
// signalling NaNs of operands loaded from memory (one extra instruction per
// operand); the weights are finite, so that step is skipped here.  The
// results only feed ordinary instructions (never a DPP or lane read directly).
__device__ __forceinline__ uint32_t pk_min_raw(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_min_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ uint32_t pk_max_raw(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_max_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}

// (min, -max) of a chunk's 8 fp16 values as an fp16 pair: taking -max lets
// one packed minimum reduce both extrema.  Comparisons of fp16 values are
// exact, so these are the very values an fp32 comparison would select.
__device__ __forceinline__ uint32_t chunk_extrema(const u4_t& d) {
  const uint32_t lo = pk_min_raw(pk_min_raw(d[0], d[1]), pk_min_raw(d[2], d[3]));
  const uint32_t hi = pk_max_raw(pk_max_raw(d[0], d[1]), pk_max_raw(d[2], d[3]));
  const h2_t l = as_h2(lo), h = as_h2(hi);
  h2_t r;
  r.x = __builtin_elementwise_min(l.x, l.y);
  r.y = -__builtin_elementwise_max(h.x, h.y);
  return as_u32(r);
}

// Reduce (min, -max) pairs over aligned groups of 4, 8 or 16 lanes.
__device__ __forceinline__ uint32_t reduce_lanes16(uint32_t p, int lanes) {
  p = pk_min(p, dpp<0xb1>(p));                  // quad_perm [1,0,3,2]
  p = pk_min(p, dpp<0x4e>(p));                  // quad_perm [2,3,0,1]
  if (lanes >= 8) p = pk_min(p, dpp<0x141>(p));   // row_half_mirror
  if (lanes >= 16) p = pk_min(p, dpp<0x140>(p));  // row_mirror
  return p;
}

// Over the whole wave; every lane receives the result.
__device__ __forceinline__ uint32_t reduce_wave(uint32_t p) {
  p = reduce_lanes16(p, 16);
  const uint32_t a = pk_min((uint32_t)__builtin_amdgcn_readlane((int)p, 0),
                            (uint32_t)__builtin_amdgcn_readlane((int)p, 16));
  const uint32_t b = pk_min((uint32_t)__builtin_amdgcn_readlane((int)p, 32),
                            (uint32_t)__builtin_amdgcn_readlane((int)p, 48));
  return pk_min(a, b);
}

// Scale, zero point and the two-term reciprocal of the scale of one group.
struct Params {
  float r_hi, r_lo;  // r_hi + r_lo = 1/s
  uint32_t zz;       // z - kRoundBits (mod 2^32): folds the rounding offset into the zero
  uint32_t s16;      // stored scale (fp16 bits)
  int z;             // stored zero point
  int qlo;           // lowest code: 0 (min-max grid) or 1 (signed symmetric grid)
};

// The fp32 quotient x / D for a small constant divisor D, correctly rounded
// (the two-term reciprocal form, checked for every fp32 significand and
// D = 3, 7, 15, 127, 255; D = 1 is exact).
template <int D>
__device__ __forceinline__ float div_const(float x) {
  constexpr float m_hi = 1.0f / (float)D;
  constexpr float m_lo = (float)((1.0 - (double)D * (double)m_hi) * (double)m_hi);
  return __builtin_fmaf(x, m_hi, x * m_lo);
}

// Min-max grid: scale = fp16((max - min) / M), zero = rint(-min / scale).
// Signed symmetric grid (SYM): scale = fp16(max|w| / qmax), qmax =
// 2^(b-1) - 1, zero = 2^(b-1), codes from 1.  A zero scale becomes 1.  Every
// quotient equals the correctly rounded fp32 one.
template <int BITS>
__device__ __forceinline__ Params group_params(uint32_t ext, bool sym) {
  constexpr int M = (1 << BITS) - 1;
  constexpr int QMAX = (1 << (BITS - 1)) - 1;
  const h2_t e = as_h2(ext);
  const float lo = (float)e.x;
  const float hi = -(float)e.y;
  float s32 = sym ? div_const<QMAX>(fmaxf(-lo, hi)) : div_const<M>(hi - lo);
  // The scale is rounded twice: to fp32 (the quotient), then to fp16.  This
  // empty barrier keeps the fp32 value: otherwise the fma and the conversion
  // are folded into one mixed-precision fma that rounds once, straight to
  // fp16, which differs when the fp32 quotient is an fp16 halfway case.
  asm("" : "+v"(s32));
  uint32_t s16 = f32_to_h_bits(s32);
  if ((s16 & 0x7fffu) == 0) s16 = 0x3c00u;
  const float s = h_bits_to_f32((uint16_t)s16);
  Params p;
  p.r_hi = 1.0f / s;
  p.r_lo = __builtin_fmaf(-s, p.r_hi, 1.0f) * p.r_hi;
  const float nl = -lo;
  p.z = sym ? 1 << (BITS - 1) : (int)__builtin_rintf(__builtin_fmaf(nl, p.r_hi, nl * p.r_lo));
  p.zz = (uint32_t)p.z - kRoundBits;
  p.s16 = s16;
  p.qlo = sym ? 1 : 0;
  return p;
}

// q = clamp(rint(w / s) + z, qlo, M) for one fp16 weight.
template <int BITS>
__device__ __forceinline__ uint32_t code_of(_Float16 wh, const Params& p) {
  constexpr int M = (1 << BITS) - 1;
  const float w = (float)wh;
  // w * r_lo written as an fma with a zero addend so that it, too, takes the
  // fp16 weight directly (the sign of a zero product cannot change the code)
  const float v = __builtin_fmaf(w, p.r_hi, __builtin_fmaf(w, p.r_lo, 0.0f));
  const uint32_t t = __builtin_bit_cast(uint32_t, v + kRoundMagic) + p.zz;
  return (uint32_t)min(max((int)t, p.qlo), M);
}

// The 8 codes of a chunk, packed least significant first (8-bit codes do not
// fit one word: their packed form is code_bytes).
template <int BITS>
__device__ __forceinline__ uint32_t chunk_codes(const u4_t& d, const Params& p, uint32_t (&q)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const h2_t v = as_h2(d[i]);
    q[2 * i] = code_of<BITS>(v.x, p);
    q[2 * i + 1] = code_of<BITS>(v.y, p);
  }
  uint32_t acc = 0;
  if constexpr (BITS < 8) {
    acc = q[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) acc |= q[i] << (BITS * i);
  }
  return acc;
}

__device__ __forceinline__ u2_t code_bytes(const uint32_t (&q)[8]) {
  u2_t b;
  b[0] = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
  b[1] = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
  return b;
}

// Byte offset (within the row's packed words) of what this thread stores for
// its chunk c = t (add `step` per further round of T chunks).  For 3-bit codes
// the four lanes of a quad hold chunks 4m..4m+3, one 96-bit period: lane
// j < 3 stores word j of the period; lane 3 gets an offset far past any row,
// so the buffer unit drops its store.
template <int BITS>
struct StoreMap {
  uint32_t off, step, shift;
  __device__ __forceinline__ StoreMap(uint32_t t, uint32_t T) {
    if constexpr (BITS == 8) {
      off = t * 8u;
      step = T * 8u;
    } else if constexpr (BITS == 4) {
      off = t * 4u;
      step = T * 4u;
    } else if constexpr (BITS == 2) {
      off = t * 2u;
      step = T * 2u;
    } else {
      const uint32_t j = t & 3u;
      off = j < 3u ? (3u * (t >> 2) + j) * 4u : 0x80000000u;
      step = T * 3u;
      shift = 8u + 8u * j;
    }
  }
};

// Store a chunk's packed codes (`bits` holds its 8*BITS bits).  Every lane
// of a quad must be active (3-bit codes exchange bits with the right
// neighbour).  Stores past the buffer's end are dropped by the buffer unit.
template <int BITS>
__device__ __forceinline__ void store_chunk(__amdgpu_buffer_rsrc_t prs, uint32_t bits,
                                            const StoreMap<BITS>& m, uint32_t i) {
  const uint32_t off = m.off + i * m.step;
  if constexpr (BITS == 4) {
    __builtin_amdgcn_raw_buffer_store_b32(bits, prs, (int)off, 0, 0);
  } else if constexpr (BITS == 2) {
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)bits, prs, (int)off, 0, 0);
  } else {
    const uint32_t next = dpp<0xf9>(bits);  // quad_perm [1,2,3,3]
    const uint32_t word = __builtin_amdgcn_alignbit(next, bits << 8, m.shift);
    __builtin_amdgcn_raw_buffer_store_b32(word, prs, (int)off, 0, 0);
  }
}

// One workgroup of T = blockDim.x threads per row; thread t owns chunks
// c = i*T + t, i < NL.  Chunks past the row's end load zeros (buffer range
// check), take no part in the extrema and store nothing.
template <int BITS, int NL, int MODE, bool CODES>
__global__ __launch_bounds__(1024) void rtn_quantize_kernel(
    const uint16_t* __restrict__ w, int K, int G, int cpg /* chunks per group */,
    int lg_cpg /* log2(cpg) when MODE == kLaneGroups */, int sym, uint8_t* __restrict__ codes,
    uint32_t* __restrict__ packed, uint16_t* __restrict__ scales, int32_t* __restrict__ zeros) {
  extern __shared__ uint32_t ent[];  // kLdsGroups: one (min, -max) pair per chunk

  const int T = blockDim.x;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t >> 6;
  const int waves = T >> 6;
  const uint32_t C = (uint32_t)K >> 3;
  const int64_t row = blockIdx.x;
  const auto wrs = rsrc(w + row * K, (uint32_t)K * 2u);
  const uint32_t row_words = (uint32_t)K * BITS / 32u;
  const auto prs = rsrc(packed + row * row_words, packed ? row_words * 4u : 0u);
  const auto crs = rsrc(codes + row * K, codes ? (uint32_t)K : 0u);

  u4_t d[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i)
    d[i] = __builtin_amdgcn_raw_buffer_load_b128(wrs, (int)((uint32_t)(i * T + t) * 16u), 0, kSlc);

  // Codes of chunk i.  Without a packed output the buffer range is empty and
  // the packed stores are dropped; byte codes are a compile-time choice.
  const StoreMap<BITS> smap((uint32_t)t, (uint32_t)T);
  auto emit = [&](int i, const Params& p) {
    uint32_t q[8];
    const uint32_t bits = chunk_codes<BITS>(d[i], p, q);
    if constexpr (CODES)
      __builtin_amdgcn_raw_buffer_store_b64(code_bytes(q), crs, (int)((uint32_t)(i * T + t) * 8u),
                                            0, 0);
    if constexpr (BITS == 8)
      __builtin_amdgcn_raw_buffer_store_b64(code_bytes(q), prs,
                                            (int)(smap.off + (uint32_t)i * smap.step), 0, 0);
    else
      store_chunk<BITS>(prs, bits, smap, (uint32_t)i);
  };

  if constexpr (MODE == kRowGroup) {
    __shared__ uint32_t wave_ext[16];
    uint32_t lo = kPosInfPair, hi = kPosInfPair ^ 0x80008000u;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      if ((uint32_t)(i * T + t) < C) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          lo = pk_min_raw(lo, d[i][k]);
          hi = pk_max_raw(hi, d[i][k]);
        }
      }
    }
    const h2_t l = as_h2(lo), h = as_h2(hi);
    h2_t e;
    e.x = __builtin_elementwise_min(l.x, l.y);
    e.y = -__builtin_elementwise_max(h.x, h.y);
    uint32_t ext = reduce_wave(as_u32(e));
    if (waves > 1) {
      if (lane == 0) wave_ext[wave] = ext;
      __syncthreads();
      ext = wave_ext[0];
      for (int k = 1; k < waves; ++k) ext = pk_min(ext, wave_ext[k]);
    }
    const Params p = group_params<BITS>(ext, sym != 0);
    if (t == 0) {
      scales[row] = (uint16_t)p.s16;
      zeros[row] = p.z;
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) emit(i, p);
  } else if constexpr (MODE == kLaneGroups) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const uint32_t c = (uint32_t)(i * T + t);
      uint32_t ext = reduce_lanes16(chunk_extrema(d[i]), cpg);
      if (cpg >= 32) ext = pk_min(ext, (uint32_t)__builtin_amdgcn_ds_swizzle((int)ext, 0x401F));
      if (cpg >= 64)
        ext = pk_min((uint32_t)__builtin_amdgcn_readlane((int)ext, 0),
                     (uint32_t)__builtin_amdgcn_readlane((int)ext, 32));
      const Params p = group_params<BITS>(ext, sym != 0);
      if ((lane & (cpg - 1)) == 0 && c < C) {
        const int64_t j = row * G + (c >> lg_cpg);
        scales[j] = (uint16_t)p.s16;
        zeros[j] = p.z;
      }
      emit(i, p);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const uint32_t c = (uint32_t)(i * T + t);
      if (c < C) ent[c] = chunk_extrema(d[i]);
    }
    __syncthreads();
    // A wave per group.  Its three parameters then overwrite the group's
    // first entries (cpg >= 12 here), which only this wave reads.
    for (int j = wave; j < G; j += waves) {
      uint32_t ext = kPosInfPair;
      for (int e = lane; e < cpg; e += kWave) ext = pk_min(ext, ent[j * cpg + e]);
      ext = reduce_wave(ext);
      const Params p = group_params<BITS>(ext, sym != 0);
      if (lane == 0) {
        scales[row * G + j] = (uint16_t)p.s16;
        zeros[row * G + j] = p.z;
        ent[j * cpg] = __builtin_bit_cast(uint32_t, p.r_hi);
        ent[j * cpg + 1] = __builtin_bit_cast(uint32_t, p.r_lo);
        ent[j * cpg + 2] = p.zz;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const uint32_t c = (uint32_t)(i * T + t);
      const uint32_t j = min(c / (uint32_t)cpg, (uint32_t)G - 1u);
      Params p;
      p.r_hi = __builtin_bit_cast(float, ent[j * cpg]);
      p.r_lo = __builtin_bit_cast(float, ent[j * cpg + 1]);
      p.zz = ent[j * cpg + 2];
      p.qlo = sym ? 1 : 0;
      emit(i, p);
    }
  }
}

// Packs byte codes: chunk c of the whole [N][K] matrix (8 codes, one 64-bit
// load) lands at the same place of the concatenated packed rows, because
// every row holds a whole number of chunks and (for 3-bit) of 4-chunk periods.
template <int BITS>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ codes,
                                                   int64_t nchunks, uint32_t* __restrict__ packed) {
  constexpr uint32_t mask = (1u << BITS) - 1u;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // nchunks is a multiple of 4, so quads of lanes are active or idle together
  for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < nchunks; c += stride) {
    const u2_t b = *reinterpret_cast<const u2_t*>(codes + 8 * c);
    if constexpr (BITS == 8) {  // code k is byte k of the row: a copy
      reinterpret_cast<u2_t*>(packed)[c] = b;
      continue;
    }
    uint32_t bits = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) bits |= ((b[i >> 2] >> (8 * (i & 3))) & mask) << (BITS * i);
    if constexpr (BITS == 4) {
      packed[c] = bits;
    } else if constexpr (BITS == 2) {
      reinterpret_cast<uint16_t*>(packed)[c] = (uint16_t)bits;
    } else {
      const uint32_t next = dpp<0xf9>(bits);  // quad_perm [1,2,3,3]
      const uint32_t j = (uint32_t)lane & 3u;
      const uint32_t word = __builtin_amdgcn_alignbit(next, bits << 8, 8u + 8u * j);
      if (j < 3u) packed[3 * (c >> 2) + j] = word;
    }
  }
}

// Compact group words: fp16 scale bits | int16 zero point << 16, the zero
// saturated to the int16 range; each wave adds its saturation count to
// *saturated once.
__global__ __launch_bounds__(256) void pack_meta_kernel(const uint16_t* __restrict__ scales,
                                                        const int32_t* __restrict__ zeros,
                                                        int64_t count, uint32_t* __restrict__ meta,
                                                        int32_t* __restrict__ saturated) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int sat = 0;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < count; i += stride) {
    const int32_t z = zeros[i];
    const int32_t zc = min(max(z, -32768), 32767);
    sat += zc != z ? 1 : 0;
    meta[i] = (uint32_t)scales[i] | ((uint32_t)(uint16_t)(int16_t)zc << 16);
  }
  if (saturated) {
    for (int o = kWave / 2; o > 0; o >>= 1) sat += __shfl_xor(sat, o);
    if ((threadIdx.x & (kWave - 1)) == 0 && sat != 0) atomicAdd(saturated, sat);
  }
}

constexpr int kChunkCounts[] = {1, 2, 4, 6, 8, 16};

template <int BITS, int MODE>
hipError_t launch_mode(const uint16_t* w, int64_t N, int K, int G, int cpg, int lg_cpg, int T,
                       int nl, size_t lds, int sym, uint8_t* codes, uint32_t* packed,
                       uint16_t* scales, int32_t* zeros, hipStream_t stream) {
  const dim3 grid((unsigned)N), block((unsigned)T);
#define LOWBIT_Q_NL(n)                                                                      \
  case n:                                                                                   \
    if (codes)                                                                              \
      hipLaunchKernelGGL((rtn_quantize_kernel<BITS, n, MODE, true>), grid, block, lds, stream, \
                         w, K, G, cpg, lg_cpg, sym, codes, packed, scales, zeros);               \
    else                                                                                    \
      hipLaunchKernelGGL((rtn_quantize_kernel<BITS, n, MODE, false>), grid, block, lds,       \
                         stream, w, K, G, cpg, lg_cpg, sym, codes, packed, scales, zeros);       \
    break;
  switch (nl) {
    LOWBIT_Q_NL(1)
    LOWBIT_Q_NL(2)
    LOWBIT_Q_NL(4)
    LOWBIT_Q_NL(6)
    LOWBIT_Q_NL(8)
    LOWBIT_Q_NL(16)
    default:
      return hipErrorInvalidValue;
  }
#undef LOWBIT_Q_NL
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(const uint16_t* w, int64_t N, int K, int G, int cpg, int T, int nl,
                       int sym, uint8_t* codes, uint32_t* packed, uint16_t* scales,
                       int32_t* zeros, hipStream_t stream) {
  const bool pow2 = (cpg & (cpg - 1)) == 0;
  if (G == 1)
    return launch_mode<BITS, kRowGroup>(w, N, K, G, cpg, 0, T, nl, 0, sym, codes, packed,
                                        scales, zeros, stream);
  if (pow2 && cpg <= kWave) {
    int lg = 0;
    while ((1 << lg) < cpg) ++lg;
    return launch_mode<BITS, kLaneGroups>(w, N, K, G, cpg, lg, T, nl, 0, sym, codes, packed,
                                          scales, zeros, stream);
  }
  const size_t lds = (size_t)(K / 8) * 4;
  return launch_mode<BITS, kLdsGroups>(w, N, K, G, cpg, 0, T, nl, lds, sym, codes, packed,
                                       scales, zeros, stream);
}

}  // namespace

hipError_t launch_quantize(const uint16_t* w, int64_t N, int64_t K, int bits, int64_t gsz,
                           bool sym, uint8_t* codes, uint32_t* packed, uint16_t* scales,
                           int32_t* zeros, hipStream_t stream) {
  const int64_t g = gsz == 0 ? K : gsz;
  const int G = (int)(K / g);
  const int cpg = (int)(g / 8);
  const int64_t C = K / 8;
  // Threads per row: enough that a thread owns at most 8 chunks (16 when the
  // 1024-thread limit binds); at least one wave.
  int T = kWave;
  while (T < 1024 && (int64_t)T * 8 < C) T *= 2;
  const int need = (int)((C + T - 1) / T);
  int nl = 0;
  for (int n : kChunkCounts)
    if (n >= need) {
      nl = n;
      break;
    }
  if (nl == 0) return hipErrorInvalidValue;
  switch (bits) {
    case 2:
      return launch_bits<2>(w, N, (int)K, G, cpg, T, nl, sym ? 1 : 0, codes, packed, scales, zeros,
                            stream);
    case 3:
      return launch_bits<3>(w, N, (int)K, G, cpg, T, nl, sym ? 1 : 0, codes, packed, scales, zeros,
                            stream);
    case 8:
      return launch_bits<8>(w, N, (int)K, G, cpg, T, nl, sym ? 1 : 0, codes, packed, scales, zeros,
                            stream);
    default:
      return launch_bits<4>(w, N, (int)K, G, cpg, T, nl, sym ? 1 : 0, codes, packed, scales, zeros,
                            stream);
  }
}

hipError_t launch_pack_meta(const uint16_t* scales, const int32_t* zeros, int64_t count,
                            uint32_t* meta, int32_t* saturated, hipStream_t stream) {
  const int64_t want = (count + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  const dim3 grid((unsigned)(want < cap ? want : cap)), block(256);
  hipLaunchKernelGGL(pack_meta_kernel, grid, block, 0, stream, scales, zeros, count, meta,
                     saturated);
  return hipGetLastError();
}

hipError_t launch_pack(const uint8_t* codes, int64_t N, int64_t K, int bits, uint32_t* packed,
                       hipStream_t stream) {
  const int64_t nchunks = N * (K / 8);
  const int64_t want = (nchunks + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 16;
  const dim3 grid((unsigned)(want < cap ? want : cap)), block(256);
  switch (bits) {
    case 2:
      hipLaunchKernelGGL(pack_kernel<2>, grid, block, 0, stream, codes, nchunks, packed);
      break;
    case 3:
      hipLaunchKernelGGL(pack_kernel<3>, grid, block, 0, stream, codes, nchunks, packed);
      break;
    case 8:
      hipLaunchKernelGGL(pack_kernel<8>, grid, block, 0, stream, codes, nchunks, packed);
      break;
    default:
      hipLaunchKernelGGL(pack_kernel<4>, grid, block, 0, stream, codes, nchunks, packed);
      break;
  }
  return hipGetLastError();
}

}  // namespace lowbit
