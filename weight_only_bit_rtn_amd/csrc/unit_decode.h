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
  __device__ static __forceinline__ uint32_t magic(const uint32_t (&w)[WORDS], int s) {
    const int d = s >> 2, i = s & 3;
    const uint32_t v = (i >= 2) ? (w[d] >> 8) : w[d];
    const uint32_t mask = (i & 1) ? 0x00F000F0u : 0x000F000Fu;
    return (v & mask) | 0x64006400u;
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
  __device__ static __forceinline__ uint32_t magic(const uint32_t (&w)[WORDS], int s) {
    const int d = s >> 3, i = s & 7;
    const uint32_t v = (i < 5) ? w[d] : (w[d] >> 10);
    return (v & (0x00030003u << pos(s))) | 0x64006400u;
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
  // Ten-code windows of one 32-code period (words d0 d1 d2 = stream bits
  // 0..95): window 0 = d0 (codes 0..9 at bits 0,3,..,27), window 1 = stream
  // bits 30..61 (codes 10..19), window 2 = stream bits 60..91 (codes 20..29).
  __device__ static __forceinline__ uint32_t window(const uint32_t (&w)[WORDS], int base, int m) {
    return m == 0 ? w[base]
           : m == 1 ? __builtin_amdgcn_alignbit(w[base + 1], w[base], 30)
                    : __builtin_amdgcn_alignbit(w[base + 2], w[base + 1], 28);
  }
  __device__ static __forceinline__ uint32_t magic(const uint32_t (&w)[WORDS], int s) {
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
    return (v & (0x00070007u << pos(s))) | 0x64006400u;
  }
  __device__ static __forceinline__ uint32_t code(const uint32_t (&w)[WORDS], int c) {
    const int base = 3 * (c >> 5), bit = 3 * (c & 31), wi = bit >> 5, off = bit & 31;
    uint32_t v = w[base + wi] >> off;
    if (off > 29) v |= w[base + wi + 1] << (32 - off);
    return v & 7u;
  }
};

// Slot order must put the four slots of a quad on consecutive codes, both for
// the low and the high halves: the activation staging relies on it.
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

// Raw per-half quantization parameters (scale bits, zero, lane validity).
struct HalfParams {
  uint16_t s_lo, s_hi;
  int32_t z_lo, z_hi;
  bool v_lo, v_hi;
};

template <int BITS>
struct Consts {
  h2_t hz[Unit<BITS>::PMAX + 1];
  h2_t hs[Unit<BITS>::PMAX + 1];
};

// Can the magic-number decode reproduce fp16_rne((q - z) * s) exactly?
template <int PMAX>
__device__ __forceinline__ bool half_fast(uint16_t sb, int32_t z) {
  const int zp = z * (1 << PMAX);
  const float s = h_bits_to_f32(sb);
  const float sp = s * (1.0f / (float)(1 << PMAX));  // exact in fp32
  const float back = (float)(_Float16)sp;
  return zp >= -1024 && zp <= 1023 && back == sp;
}

template <int BITS>
__device__ __forceinline__ bool make_consts(const HalfParams& hp, Consts<BITS>& c) {
  using U = Unit<BITS>;
  constexpr int PMAX = U::PMAX;
  const float sl = h_bits_to_f32(hp.s_lo), sh = h_bits_to_f32(hp.s_hi);
#pragma unroll
  for (int p = 0; p <= PMAX; ++p) {
    if (!U::uses(p)) continue;
    const float inv = 1.0f / (float)(1 << p);
    const _Float16 hzl = (_Float16)(1024.0f + (float)(hp.z_lo * (1 << p)));
    const _Float16 hzh = (_Float16)(1024.0f + (float)(hp.z_hi * (1 << p)));
    const _Float16 hsl = hp.v_lo ? (_Float16)(sl * inv) : (_Float16)0.0f;
    const _Float16 hsh = hp.v_hi ? (_Float16)(sh * inv) : (_Float16)0.0f;
    c.hz[p] = h2_t{hzl, hzh};
    c.hs[p] = h2_t{hsl, hsh};
  }
  const bool fl = !hp.v_lo || half_fast<PMAX>(hp.s_lo, hp.z_lo);
  const bool fh = !hp.v_hi || half_fast<PMAX>(hp.s_hi, hp.z_hi);
  return fl && fh;
}

// Exact dequantized pair of slot s the slow way: extract both codes, form the
// exact product in fp64 and round it once to fp16.
template <int BITS>
__device__ __forceinline__ h2_t slow_pair(const uint32_t (&w)[Unit<BITS>::WORDS], int s,
                                          const HalfParams& hp) {
  using U = Unit<BITS>;
  const int ql = (int)U::code(w, U::lo(s));
  const int qh = (int)U::code(w, U::hi(s));
  const double sl = (double)h_bits_to_f32(hp.s_lo), sh = (double)h_bits_to_f32(hp.s_hi);
  const uint16_t dl = hp.v_lo ? f64_to_h_bits((double)(ql - hp.z_lo) * sl) : (uint16_t)0;
  const uint16_t dh = hp.v_hi ? f64_to_h_bits((double)(qh - hp.z_hi) * sh) : (uint16_t)0;
  return as_h2((uint32_t)dl | ((uint32_t)dh << 16));
}

template <int BITS>
__device__ __forceinline__ h2_t fast_pair(const uint32_t (&w)[Unit<BITS>::WORDS], int s,
                                          const Consts<BITS>& c) {
  using U = Unit<BITS>;
  const h2_t m = as_h2(U::magic(w, s));
  return (m - c.hz[U::pos(s)]) * c.hs[U::pos(s)];
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
