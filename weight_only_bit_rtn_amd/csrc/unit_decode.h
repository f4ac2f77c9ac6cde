// unit_decode.h -- turning packed b-bit codes into exact fp16 dequantized pairs.
//
// The product y = x * deq(W)^T needs, per weight, deq = fp16_rne((q - z) * s)
// computed exactly (the stored-fp16 scale and integer zero of min-max RTN:
// BladeLLM model quantization, "Quantization algorithms", MinMax; OPTQ
// reproducibility card, "Experiment Setup" row).  The decode works on
// "units": the packed bits one lane loads at once.
//
//   4-bit: one 32-code period, 4 words (one 16-byte load)
//   2-bit: two consecutive periods, 64 codes, 4 words (one 16-byte load)
//   3-bit: two periods a and b taken from different places of the row,
//          3 words each (two 12-byte loads)
//   8-bit: 16 codes, 4 words (one 16-byte load)
//
// A unit yields 16 or 32 "slots": pairs of codes (lo, hi) that end up in the
// low and high fp16 halves of one 32-bit register, so that the fp16 math runs
// two codes per instruction.  A slot's code field sits at bit position p of
// both halves; OR-ing it into the fp16 pattern of 1024 (0x6400) gives the
// exact fp16 value 1024 + q*2^p ("magic number" conversion), then
//
//   deq = ((1024 + q*2^p) - (1024 + z*2^p)) * (s*2^-p)
//
// where the subtraction is exact (both operands are integers below 2048) and
// the product (q - z) * 2^p * s * 2^-p = (q - z) * s is rounded once, by the
// fp16 multiply.  This is exact whenever 1024 + z*2^p is an integer in
// [0, 2047] and s*2^-p is an fp16 number; the per-group check below tests
// both, and groups that fail it take a slower per-code path that computes
// the exact product in fp64 and rounds it to fp16 directly.
//
// The activations are stored on chip in the same slot order, so no
// per-weight shuffle is needed in the inner loop.
//
// 8-bit codes cannot use a shifted field (1024 + q*2^p stays below 2048 only
// for p = 0), so each slot pairs two neighbouring bytes of one word and a
// single byte permute drops them under the two 0x64 exponent bytes of the
// magic register: p = 0 for every slot.
#pragma once

#include "common.h"

namespace lowbit {

template <int BITS>
struct Unit;

template <>
struct Unit<4> {
  static constexpr int CODES = 32, WORDS = 4, SLOTS = 16, QUADS = 4, PMAX = 4;
  static constexpr int NCONST = 1;  // constant sets per unit
  __host__ __device__ static constexpr int lo(int s) { return 8 * (s >> 2) + (s & 3); }
  __host__ __device__ static constexpr int hi(int s) { return lo(s) + 4; }
  __host__ __device__ static constexpr int pos(int s) { return (s & 1) ? 4 : 0; }
  __host__ __device__ static constexpr int cset(int) { return 0; }
  __host__ __device__ static constexpr bool uses(int p) { return p == 0 || p == 4; }
  static constexpr int NPOS = 2;  // distinct bit positions p, indexed by pidx
  __host__ __device__ static constexpr int pidx(int p) { return p >> 2; }
  __device__ static __forceinline__ uint32_t magic(const uint32_t (&w)[WORDS], int s,
                                                    uint32_t mg) {
    const int d = s >> 2, i = s & 3;
    const uint32_t v = (i >= 2) ? (w[d] >> 8) : w[d];
    const uint32_t mask = (i & 1) ? 0x00F000F0u : 0x000F000Fu;
    return (v & mask) | mg;
  }
  __device__ static __forceinline__ uint32_t code(const uint32_t (&w)[WORDS], int c) {
    return (w[c >> 3] >> (4 * (c & 7))) & 15u;
  }
};

template <>
struct Unit<2> {
  static constexpr int CODES = 64, WORDS = 4, SLOTS = 32, QUADS = 8, PMAX = 8;
  static constexpr int NCONST = 2;  // the two periods may sit in different groups
  __host__ __device__ static constexpr int lo(int s) { return 16 * (s >> 3) + (s & 7); }
  __host__ __device__ static constexpr int hi(int s) { return lo(s) + 8; }
  __host__ __device__ static constexpr int pos(int s) {
    return (s & 7) < 5 ? 2 * (s & 7) : 2 * ((s & 7) - 5);
  }
  __host__ __device__ static constexpr int cset(int s) { return s >> 4; }
  __host__ __device__ static constexpr bool uses(int p) { return p <= 8 && (p & 1) == 0; }
  static constexpr int NPOS = 5;
  __host__ __device__ static constexpr int pidx(int p) { return p >> 1; }
  __device__ static __forceinline__ uint32_t magic(const uint32_t (&w)[WORDS], int s,
                                                    uint32_t mg) {
    const int d = s >> 3, i = s & 7;
    const uint32_t v = (i < 5) ? w[d] : (w[d] >> 10);
    return (v & (0x00030003u << pos(s))) | mg;
  }
  __device__ static __forceinline__ uint32_t code(const uint32_t (&w)[WORDS], int c) {
    return (w[c >> 4] >> (2 * (c & 15))) & 3u;
  }
};

template <>
struct Unit<3> {
  static constexpr int CODES = 64, WORDS = 6, SLOTS = 32, QUADS = 8, PMAX = 7;
  static constexpr int NCONST = 1;  // per-half constants: lo half = period a, hi = period b
  __host__ __device__ static constexpr int lo(int s) { return s; }
  __host__ __device__ static constexpr int hi(int s) { return 32 + s; }
  __host__ __device__ static constexpr int pos(int s) {
    // slots 10m+i take code i of the m-th ten-code window; 30, 31 the last two codes
    return s < 30 ? ((s % 10) == 0 || (s % 10) == 8 ? 0
                     : (s % 10) == 1 || (s % 10) == 9 ? 3
                     : (s % 10) == 2 ? 6
                     : (s % 10) == 3 ? 1
                     : (s % 10) == 4 ? 4
                     : (s % 10) == 5 ? 7
                     : (s % 10) == 6 ? 2
                                     : 5)
                  : (s == 30 ? 2 : 5);
  }
  __host__ __device__ static constexpr int cset(int) { return 0; }
  __host__ __device__ static constexpr bool uses(int p) { return p <= 7; }
  static constexpr int NPOS = 8;
  __host__ __device__ static constexpr int pidx(int p) { return p; }
  // Ten-code windows of one 32-code period (words d0 d1 d2 = stream bits
  // 0..95): window 0 = d0 (codes 0..9 at bits 0,3,..,27), window 1 = stream
  // bits 30..61 (codes 10..19), window 2 = stream bits 60..91 (codes 20..29).
  __device__ static __forceinline__ uint32_t window(const uint32_t (&w)[WORDS], int base, int m) {
    return m == 0 ? w[base]
           : m == 1 ? __builtin_amdgcn_alignbit(w[base + 1], w[base], 30)
                    : __builtin_amdgcn_alignbit(w[base + 2], w[base + 1], 28);
  }
  __device__ static __forceinline__ uint32_t magic(const uint32_t (&w)[WORDS], int s,
                                                    uint32_t mg) {
    uint32_t v;
    if (s < 30) {
      const int m = s / 10, i = s % 10;
      const uint32_t ua = window(w, 0, m), ub = window(w, 3, m);
      // byte windows: 16 bits of period a in the low half, the same 16 bits
      // of period b in the high half (v_perm_b32 byte select; 0x0c = zero)
      const uint32_t sel = i < 3 ? 0x05040100u : i < 6 ? 0x06050201u : i < 8 ? 0x07060302u
                                                                         : 0x0c070c03u;
      v = __builtin_amdgcn_perm(ub, ua, sel);
    } else {
      // codes 30, 31 sit in bits 26..31 of d2: take byte 3 of each period
      v = __builtin_amdgcn_perm(w[5], w[2], 0x0c070c03u);
    }
    return (v & (0x00070007u << pos(s))) | mg;
  }
  __device__ static __forceinline__ uint32_t code(const uint32_t (&w)[WORDS], int c) {
    const int base = 3 * (c >> 5), bit = 3 * (c & 31), wi = bit >> 5, off = bit & 31;
    uint32_t v = w[base + wi] >> off;
    if (off > 29) v |= w[base + wi + 1] << (32 - off);
    return v & 7u;
  }
};

template <>
struct Unit<8> {
  static constexpr int CODES = 16, WORDS = 4, SLOTS = 8, QUADS = 2, PMAX = 0;
  static constexpr int NCONST = 1;
  // slot s: codes 2s (low half) and 2s + 1 (high half), bytes 0, 1 (s even)
  // or 2, 3 (s odd) of word s / 2; a quad is eight consecutive codes
  __host__ __device__ static constexpr int lo(int s) { return 2 * s; }
  __host__ __device__ static constexpr int hi(int s) { return 2 * s + 1; }
  __host__ __device__ static constexpr int pos(int) { return 0; }
  __host__ __device__ static constexpr int cset(int) { return 0; }
  __host__ __device__ static constexpr bool uses(int p) { return p == 0; }
  static constexpr int NPOS = 1;
  __host__ __device__ static constexpr int pidx(int) { return 0; }
  // v_perm_b32 selectors 0..3 pick bytes of the word, 4..7 bytes of the magic
  // register 0x64006400 (5 and 7 are its 0x64 bytes)
  __device__ static __forceinline__ uint32_t magic(const uint32_t (&w)[WORDS], int s,
                                                    uint32_t mg) {
    return __builtin_amdgcn_perm(mg, w[s >> 1], (s & 1) ? 0x07030502u : 0x07010500u);
  }
  __device__ static __forceinline__ uint32_t code(const uint32_t (&w)[WORDS], int c) {
    return (w[c >> 2] >> (8 * (c & 3))) & 255u;
  }
};

// Slot order must put the four slots of a quad on consecutive codes, both for
// the low and the high halves: the activation staging relies on it (8-bit
// quads are eight consecutive codes in natural order, staged as they are).
template <int BITS>
constexpr bool quads_are_runs() {
  using U = Unit<BITS>;
  for (int q = 0; q < U::QUADS; ++q)
    for (int e = 0; e < 4; ++e)
      if (U::lo(4 * q + e) != U::lo(4 * q) + e || U::hi(4 * q + e) != U::hi(4 * q) + e)
        return false;
  return true;
}
static_assert(quads_are_runs<2>() && quads_are_runs<3>() && quads_are_runs<4>(),
              "slot order breaks the activation staging");

// Group parameters of one weight row: a scale array and a zero array, or
// (META) one compact word per group with the fp16 scale in bits 0..15 and the
// zero point as a 16-bit two's-complement integer in bits 16..31.  With META
// the words arrive through the `scales` pointer and `zeros` is unused.
template <bool META>
struct RowParams {
  const uint16_t* s = nullptr;
  const int32_t* z = nullptr;
  const uint32_t* m = nullptr;
  __device__ __forceinline__ RowParams(const uint16_t* scales, const int32_t* zeros, int64_t n,
                                       int G) {
    if constexpr (META) {
      m = reinterpret_cast<const uint32_t*>(scales) + n * G;
    } else {
      s = scales + n * G;
      z = zeros + n * G;
    }
  }
  __device__ __forceinline__ void at(int g, uint16_t& sb, int32_t& zz) const {
    if constexpr (META) {
      const uint32_t v = m[g];
      sb = (uint16_t)v;
      zz = (int32_t)v >> 16;
    } else {
      sb = s[g];
      zz = z[g];
    }
  }
};

// Raw per-half quantization parameters (scale bits, zero, lane validity).
struct HalfParams {
  uint16_t s_lo, s_hi;
  int32_t z_lo, z_hi;
  bool v_lo, v_hi;
};

// Decode constants of one unit, indexed by bit position (pidx).
//  hz[i] = 1024 + z * 2^p                          (both modes)
//  hs[i] = s * 2^-p   (scaled mode: one accumulator per output)
//  hs[0] = s          (per-position mode: the product comes out scaled by 2^p
//                      and is accumulated separately per p, rescaled at the end)
template <int BITS>
struct Consts {
  h2_t hz[Unit<BITS>::NPOS];
  h2_t hs[Unit<BITS>::NPOS];
};

// Constants from integer operations on the bit patterns (so uniform inputs
// stay in scalar registers):
//  - 1024 + z*2^p for 0 <= z*2^p < 1024 is the fp16 pattern 0x6400 | (z << p);
//  - s*2^-p is s with its exponent field lowered by p, exact as long as the
//    result stays a normal number (exponent field of s above p).
// Fast decode conditions per half (both modes): 0 <= z <= 1023 >> PMAX;
//  scaled mode: exponent field of s >= PMAX + 1;
//  per-position mode: s normal and s < 8, so that (q - z) * s * 2^p stays in
//  fp16's normal range, where scaling by 2^p commutes with the rounding.
// 8-bit codes (no shifted positions): 0 <= z <= 255 and s < 256, so that
//  |q - z| * s < 65504 for every code (also for decoded words past the end of
//  a row), subnormal scales included (the single fp16 multiply rounds them
//  correctly).
template <int BITS, bool POS>
__device__ __forceinline__ bool half_fast(uint32_t sb, int32_t z) {
  constexpr int PMAX = Unit<BITS>::PMAX;
  if constexpr (BITS == 8) return (uint32_t)z <= 255u && sb < 0x5C00u;
  const bool zok = (uint32_t)z <= (1023u >> PMAX);
  const bool sok = POS ? (sb >= 0x0400u && sb < 0x4800u) : (sb >= (uint32_t)(PMAX + 1) << 10);
  return zok && sok;
}

template <int BITS, bool POS>
__device__ __forceinline__ bool make_consts(const HalfParams& hp, Consts<BITS>& c) {
  using U = Unit<BITS>;
  const uint32_t s2 = (uint32_t)hp.s_lo | ((uint32_t)hp.s_hi << 16);
  const uint32_t z2 = ((uint32_t)hp.z_lo & 0xffffu) | ((uint32_t)hp.z_hi << 16);
  const uint32_t keep = (hp.v_lo ? 0x0000ffffu : 0u) | (hp.v_hi ? 0xffff0000u : 0u);
#pragma unroll
  for (int p = 0; p <= U::PMAX; ++p) {
    if (!U::uses(p)) continue;
    const int i = U::pidx(p);
    c.hz[i] = as_h2(0x64006400u + (z2 << p));
    if (!POS) c.hs[i] = as_h2((s2 - ((uint32_t)p << 10) * 0x10001u) & keep);
  }
  if (POS) c.hs[0] = as_h2(s2 & keep);
  const bool fl = !hp.v_lo || half_fast<BITS, POS>(hp.s_lo, hp.z_lo);
  const bool fh = !hp.v_hi || half_fast<BITS, POS>(hp.s_hi, hp.z_hi);
  return fl && fh;
}

// fp16_rne((q - z) * s) for any code, zero point and scale: the product is
// formed in fp32 and rounded to odd (its last bit records inexactness), which
// makes the following fp32 -> fp16 rounding the correctly rounded result
// (fp32 carries at least two more bits than fp16).
__device__ __forceinline__ uint16_t exact_deq(int q, int z, float s) {
  const float qz = (float)(q - z);  // exact: |q - z| < 2^24
  const float p = qz * s;
  const float e = __builtin_fmaf(qz, s, -p);  // exact remainder of the product
  uint32_t pb = __builtin_bit_cast(uint32_t, p);
  if (e != 0.0f && (pb & 1u) == 0u) pb += ((e > 0.0f) == (p > 0.0f)) ? 1u : 0xffffffffu;
  return f32_to_h_bits(__builtin_bit_cast(float, pb));
}

template <int BITS>
__device__ __forceinline__ h2_t slow_pair(const uint32_t (&w)[Unit<BITS>::WORDS], int s,
                                          const HalfParams& hp) {
  using U = Unit<BITS>;
  const int ql = (int)U::code(w, U::lo(s));
  const int qh = (int)U::code(w, U::hi(s));
  const uint16_t dl = hp.v_lo ? exact_deq(ql, hp.z_lo, h_bits_to_f32(hp.s_lo)) : (uint16_t)0;
  const uint16_t dh = hp.v_hi ? exact_deq(qh, hp.z_hi, h_bits_to_f32(hp.s_hi)) : (uint16_t)0;
  return as_h2((uint32_t)dl | ((uint32_t)dh << 16));
}

// Code c of a unit whose words are stored column-wise in LDS (word i of lane
// l at w[i * 64 + l]); c may be a run-time value.
template <int BITS>
__device__ __forceinline__ uint32_t unit_code_lds(const uint32_t* w, int lane, int c) {
  int bit;
  if constexpr (BITS == 3)
    bit = 96 * (c >> 5) + 3 * (c & 31);
  else
    bit = BITS * c;
  const int wi = bit >> 5, off = bit & 31;
  uint32_t v = w[wi * 64 + lane] >> off;
  if (off + BITS > 32) v |= w[(wi + 1) * 64 + lane] << (32 - off);
  return v & ((1u << BITS) - 1u);
}

// The fp16 bit pattern of 1024.0 in both halves, held in a vector register
// (the kernels hide its value from the compiler once, so every field
// extraction becomes a single v_and_or_b32 with the mask in a scalar register;
// gfx9 VOP3 encodings cannot carry two literals).
constexpr uint32_t kMagic1024 = 0x64006400u;

__device__ __forceinline__ uint32_t magic_register() {
  uint32_t mg = kMagic1024;
  asm volatile("" : "+v"(mg));
  return mg;
}

// Fast pair of slot s; in per-position mode the result is 2^p * deq.
template <int BITS, bool POS>
__device__ __forceinline__ h2_t fast_pair(const uint32_t (&w)[Unit<BITS>::WORDS], int s,
                                          const Consts<BITS>& c, uint32_t mg) {
  using U = Unit<BITS>;
  const int i = U::pidx(U::pos(s));
  const h2_t m = as_h2(U::magic(w, s, mg));
  return (m - c.hz[i]) * c.hs[POS ? 0 : i];
}

// Where a unit's codes live in the row.  4-bit / 2-bit units are one run of
// 32 / 64 codes starting at k = ka; a 3-bit unit is two 32-code periods
// starting at ka (codes 0..31) and kb (codes 32..63).
struct UnitRef {
  int ka, kb;    // first k of each segment
  bool va, vb;   // segment lies inside the row
};

template <int BITS>
__device__ __forceinline__ int unit_k(const UnitRef& u, int c) {
  if constexpr (BITS == 3) return c < 32 ? u.ka + c : u.kb + (c - 32);
  return u.ka + c;
}

// Load one unit's words of one row (zeros where the segment is outside).
template <int BITS>
__device__ __forceinline__ void load_unit(const uint32_t* __restrict__ rowp, const UnitRef& u,
                                          uint32_t (&w)[Unit<BITS>::WORDS]) {
  if constexpr (BITS == 3) {
    const uint32_t* pa = rowp + 3 * (u.ka >> 5);
    const uint32_t* pb = rowp + 3 * (u.kb >> 5);
    w[0] = u.va ? pa[0] : 0u;
    w[1] = u.va ? pa[1] : 0u;
    w[2] = u.va ? pa[2] : 0u;
    w[3] = u.vb ? pb[0] : 0u;
    w[4] = u.vb ? pb[1] : 0u;
    w[5] = u.vb ? pb[2] : 0u;
  } else {
    const uint4 v = u.va ? *reinterpret_cast<const uint4*>(rowp + (u.ka * BITS >> 5))
                         : make_uint4(0u, 0u, 0u, 0u);
    w[0] = v.x;
    w[1] = v.y;
    w[2] = v.z;
    w[3] = v.w;
  }
}

// Quantization parameters of constant set `cs` of a unit (per-group layout).
// Group index of input channel k: a shift when the group size is a power of
// two (gshift >= 0), a division otherwise.
__device__ __forceinline__ int group_of(int k, int gsz, int gshift) {
  return gshift >= 0 ? (k >> gshift) : k / gsz;
}

template <int BITS>
__device__ __forceinline__ HalfParams load_params(const uint16_t* __restrict__ srow,
                                                  const int32_t* __restrict__ zrow, int gsz,
                                                  int gshift, const UnitRef& u, int cs) {
  HalfParams hp;
  int kl, kh;
  bool vl, vh;
  if constexpr (BITS == 3) {
    kl = u.ka;
    kh = u.kb;
    vl = u.va;
    vh = u.vb;
  } else if constexpr (BITS == 2) {
    kl = kh = u.ka + 32 * cs;
    vl = vh = u.va;
  } else {
    kl = kh = u.ka;
    vl = vh = u.va;
  }
  const int gl = vl ? group_of(kl, gsz, gshift) : 0;
  const int gh = vh ? group_of(kh, gsz, gshift) : 0;
  hp.s_lo = srow[gl];
  hp.z_lo = zrow[gl];
  hp.s_hi = srow[gh];
  hp.z_hi = zrow[gh];
  hp.v_lo = vl;
  hp.v_hi = vh;
  return hp;
}

// One 16-byte activation entry: the four slots of quad q of a unit, each an
// fp16 pair (x[k_lo], x[k_hi]); zero where the codes lie outside the row.
template <int BITS>
__device__ __forceinline__ uint4 x_entry(const uint16_t* __restrict__ xrow, const UnitRef& u,
                                         int q, bool bvalid) {
  using U = Unit<BITS>;
  if constexpr (BITS == 8) {  // eight consecutive activations, as stored
    return (bvalid && u.va) ? *reinterpret_cast<const uint4*>(xrow + u.ka + 8 * q)
                            : make_uint4(0u, 0u, 0u, 0u);
  }
  const int c_lo = U::lo(4 * q), c_hi = U::hi(4 * q);
  const bool vl = bvalid && (BITS == 3 ? (c_lo < 32 ? u.va : u.vb) : u.va);
  const bool vh = bvalid && (BITS == 3 ? (c_hi < 32 ? u.va : u.vb) : u.va);
  const uint2 a = vl ? *reinterpret_cast<const uint2*>(xrow + unit_k<BITS>(u, c_lo))
                     : make_uint2(0u, 0u);
  const uint2 b = vh ? *reinterpret_cast<const uint2*>(xrow + unit_k<BITS>(u, c_hi))
                     : make_uint2(0u, 0u);
  return make_uint4(__builtin_amdgcn_perm(b.x, a.x, 0x05040100u),
                    __builtin_amdgcn_perm(b.x, a.x, 0x07060302u),
                    __builtin_amdgcn_perm(b.y, a.y, 0x05040100u),
                    __builtin_amdgcn_perm(b.y, a.y, 0x07060302u));
}

}  // namespace lowbit
