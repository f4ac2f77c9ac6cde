// unit_decode.h -- where the packed b-bit codes sit, and how they enter
// fp16 arithmetic.
//
// The products need, per weight, the value deq = (q - z) * s a code stands
// for (the stored fp16 scale and integer zero of min-max RTN: BladeLLM model
// quantization, "Quantization algorithms", MinMax; OPTQ reproducibility card,
// "Experiment Setup" row).  The decode works on "units": the packed bits one
// lane loads at once.
//
//   4-bit: one 32-code period, 4 words (one 16-byte load)
//   2-bit: two consecutive periods, 64 codes, 4 words (one 16-byte load)
//   3-bit: two periods a and b taken from different places of the row,
//          3 words each (two 12-byte loads)
//   8-bit: 16 codes, 4 words (one 16-byte load)
//
// A unit yields 8, 16 or 32 "slots": pairs of codes (lo, hi) that end up in
// the low and high fp16 halves of one 32-bit register, so that the fp16 math
// runs two codes per instruction.  A slot's code field sits at bit position p
// of both halves (3-bit: windows of ten codes are first cut out of the
// straddling words with funnel shifts and byte permutes).  OR-ed into the
// fp16 pattern of 2^(10 - p), the field is the exact fp16 integer
// 2^(10 - p) + q, from which one packed subtraction gives q - z exactly.
//
// The activations are stored on chip in the same slot order, so no
// per-weight shuffle is needed in the inner loop.
//
// 8-bit codes have no room for a shift (p = 0 for every slot): each slot
// pairs two neighbouring bytes of one word, which one byte permute places in
// the two halves, under the 0x64 exponent bytes of 1024.
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
  // v_perm_b32 selectors 0..3 pick bytes of the word, 4..7 bytes of mg, whose
  // bytes 1 and 3 (0x64) become the halves' high bytes: 1024 + q
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
  // NV = 2 or 4 consecutive groups g .. g + NV - 1 with one vector load per
  // array (the caller keeps g and the row's group count multiples of NV, so
  // the loads are naturally aligned and stay inside the row)
  template <int NV>
  __device__ __forceinline__ void at_vec(int g, uint16_t (&sb)[NV], int32_t (&zz)[NV]) const {
    static_assert(NV == 2 || NV == 4, "two or four groups");
    uint32_t wv[NV];
    if constexpr (META) {
      if constexpr (NV == 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(m + g);
        wv[0] = v.x, wv[1] = v.y, wv[2] = v.z, wv[3] = v.w;
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(m + g);
        wv[0] = v.x, wv[1] = v.y;
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        sb[i] = (uint16_t)wv[i];
        zz[i] = (int32_t)wv[i] >> 16;
      }
    } else {
      if constexpr (NV == 4) {
        const uint2 sv = *reinterpret_cast<const uint2*>(s + g);
        const int4 zv = *reinterpret_cast<const int4*>(z + g);
        wv[0] = sv.x, wv[1] = sv.x >> 16, wv[2] = sv.y, wv[3] = sv.y >> 16;
        zz[0] = zv.x, zz[1] = zv.y, zz[2] = zv.z, zz[3] = zv.w;
      } else {
        const uint32_t sv = *reinterpret_cast<const uint32_t*>(s + g);
        const int2 zv = *reinterpret_cast<const int2*>(z + g);
        wv[0] = sv, wv[1] = sv >> 16;
        zz[0] = zv.x, zz[1] = zv.y;
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) sb[i] = (uint16_t)wv[i];
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

// fp16 pattern of 2^(10 - p) in both halves for every field position p,
// held in vector registers (gfx9 VOP3 encodings carry no literal, and the
// field mask takes the one scalar operand, so each field extraction is one
// v_and_or_b32): OR-ed onto a field q * 2^p it gives the exact 2^(10 - p) + q.
template <int BITS>
__device__ __forceinline__ void magic_registers(uint32_t (&mgp)[Unit<BITS>::NPOS]) {
  using U = Unit<BITS>;
#pragma unroll
  for (int p = 0; p <= U::PMAX; ++p) {
    if (!U::uses(p)) continue;
    uint32_t v = (uint32_t)(25 - p) * 0x04000400u;
    asm volatile("" : "+v"(v));
    mgp[U::pidx(p)] = v;
  }
}

// Decode constants of one unit: for every field position p, the fp16 value
// 2^(10 - p) + z of each half, so that (2^(10 - p) + q) - (2^(10 - p) + z) =
// q - z exactly; and the halves' scales.
template <int BITS>
struct PConsts {
  h2_t hz[Unit<BITS>::NPOS];
  h2_t s2;
};

// The fast decode needs 2^(10 - p) + z and q - z to be fp16 integers (|z| <=
// 1024 suffices); the two-operand form (direct) also keeps (q - z) * s finite
// (0 <= s < 32, an fp16 pattern below 0x5000).  A half's two bytes of 3-bit
// units may come from different groups; other widths share one zero.
template <int BITS>
__device__ __forceinline__ bool make_pconsts(const HalfParams& hp, PConsts<BITS>& c,
                                             bool direct) {
  using U = Unit<BITS>;
  // zero points in [0, 2^(10 - PMAX)) -- those of every group whose range
  // contains 0 -- by integer operations: 2^(10 - p) + z is then the pattern
  // (25 - p) << 10 plus z << p; others by conversion (wave-uniform branch)
  const uint32_t zmax = 1024u >> U::PMAX;
  if (__all((uint32_t)hp.z_lo < zmax && (uint32_t)hp.z_hi < zmax)) {
    const uint32_t z2 = ((uint32_t)hp.z_lo & 0xffffu) | ((uint32_t)hp.z_hi << 16);
#pragma unroll
    for (int p = 0; p <= U::PMAX; ++p) {
      if (!U::uses(p)) continue;
      c.hz[U::pidx(p)] = as_h2((uint32_t)(25 - p) * 0x04000400u + (z2 << p));
    }
  } else {
#pragma unroll
    for (int p = 0; p <= U::PMAX; ++p) {
      if (!U::uses(p)) continue;
      const float base = (float)(1 << (10 - p));
      const uint32_t lo = f32_to_h_bits(base + (float)hp.z_lo);
      const uint32_t hi = BITS == 3 ? f32_to_h_bits(base + (float)hp.z_hi) : lo;
      c.hz[U::pidx(p)] = as_h2(lo | (hi << 16));
    }
  }
  c.s2 = as_h2((uint32_t)hp.s_lo | ((uint32_t)hp.s_hi << 16));
  bool ok = hp.z_lo >= -1024 && hp.z_lo <= 1024 && hp.z_hi >= -1024 && hp.z_hi <= 1024;
  if (direct) ok = ok && hp.s_lo < 0x5000u && hp.s_hi < 0x5000u;
  return ok;
}

// make_pconsts for one wave-uniform zero point z shared by both halves (one
// group per row), by scalar integer operations only, for the zero points of
// every row whose range contains 0 (0 <= z < 2^(10 - PMAX)).  Returns false
// for any other z: the caller then takes its exact per-code path (a
// conversion here would move the constants into vector registers).
template <int BITS>
__device__ __forceinline__ bool row_pconsts(int32_t z, PConsts<BITS>& c) {
  using U = Unit<BITS>;
  const uint32_t z2 = ((uint32_t)z & 0xffffu) | ((uint32_t)z << 16);
#pragma unroll
  for (int p = 0; p <= U::PMAX; ++p) {
    if (!U::uses(p)) continue;
    c.hz[U::pidx(p)] = as_h2((uint32_t)(25 - p) * 0x04000400u + (z2 << p));
  }
  return (uint32_t)z < (1024u >> U::PMAX);
}

// q - z of both codes of slot s, exact: (2^(10 - p) + q) - (2^(10 - p) + z).
template <int BITS>
__device__ __forceinline__ h2_t qz_pair(const uint32_t (&w)[Unit<BITS>::WORDS], int s,
                                        const uint32_t (&mgp)[Unit<BITS>::NPOS],
                                        const PConsts<BITS>& c) {
  using U = Unit<BITS>;
  const int i = U::pidx(U::pos(s));
  return as_h2(U::magic(w, s, mgp[i])) - c.hz[i];
}

// A value v of the exact per-code path as two fp16 numbers: its fp16
// rounding hi and the remainder lo = fp16(v - hi) (exact when v is an
// integer below 2^22 in magnitude, or an fp32 product of one with an fp16).
__device__ __forceinline__ void split_f16(float v, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_h_bits(v);
  lo = f32_to_h_bits(v - h_bits_to_f32(hi));
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

// Group index of input channel k: a shift when the group size is a power of
// two (gshift >= 0), a division otherwise.
__device__ __forceinline__ int group_of(int k, int gsz, int gshift) {
  return gshift >= 0 ? (k >> gshift) : k / gsz;
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
