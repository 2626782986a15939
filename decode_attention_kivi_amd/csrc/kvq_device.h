// Device helpers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

// fp32 -> fp16, round to nearest even (v_cvt_f16_f32 in the default mode).
__device__ __forceinline__ uint32_t f2h(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// a.lo*b.lo + a.hi*b.hi + c with fp16 pairs and an fp32 accumulator.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a),
                                __builtin_bit_cast(half2_t, b), c, false);
}

// A constant in a scalar / vector register that the compiler cannot fold
// (non-volatile, so it can still be hoisted and shared).
__device__ __forceinline__ uint32_t opaque_sgpr(uint32_t c) {
  uint32_t r;
  asm("s_mov_b32 %0, %1" : "=s"(r) : "i"(c));
  return r;
}
__device__ __forceinline__ uint32_t opaque_vgpr(uint32_t c) {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}

// Unpacking one 32-bit word of codes into fp16 pairs without conversions:
// a b-bit code moved into the fp16 mantissa under a fixed exponent reads as
// (offset + code).  Pair k of a word combines the code at bit b*k of the low
// half with the code at bit 16 + b*k of the high half.  Each pair costs one
// v_and_or_b32 (mask, exponent constant) plus the shifts that bring the codes
// into the 10 mantissa bits.
//
// NARROW layouts keep every offset <= 64 (keys: their fp32 sums include large
// outlier-channel weights, and offset * sum|weight| must stay small next to
// the logit); WIDE layouts use offsets up to 1024 and save shifts (values:
// the rounding of offset * sum(p*s) in fp32 stays far below the tolerance).
//
// The masks and exponent constants are materialized once per loop (an
// Unpacker object built outside it): routed through opaque register moves,
// they stay in registers, and instruction selection forms v_and_or_b32 (the
// gfx9-family VOP3 encoding takes no literal constant).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic) {
  return (x & mask) | magic;
}

template <int BITS, bool WIDE> struct Unpacker;

template <> struct Unpacker<2, false> {
  static constexpr int NP = 8;   // pairs per word
  uint32_t m45, m67, m89, e64, e16, e4;
  __device__ __forceinline__ Unpacker()
      : m45(opaque_sgpr(0x00300030u)), m67(opaque_sgpr(0x00C000C0u)), m89(opaque_sgpr(0x03000300u)),
        e64(opaque_vgpr(0x54005400u)), e16(opaque_vgpr(0x4C004C00u)), e4(opaque_vgpr(0x44004400u)) {}
  __device__ __forceinline__ void run(uint32_t w, uint32_t* v) const {
    const uint32_t a = w << 4, c = w >> 6;
    v[0] = and_or(a, m45, e64);  // mantissa bits 4-5: 64 + code
    v[1] = and_or(a, m67, e16);  // bits 6-7: 16 + code
    v[2] = and_or(a, m89, e4);   // bits 8-9: 4 + code
    v[3] = and_or(w, m67, e16);
    v[4] = and_or(w, m89, e4);
    v[5] = and_or(c, m45, e64);
    v[6] = and_or(c, m67, e16);
    v[7] = and_or(c, m89, e4);
  }
  __device__ static __forceinline__ float offset(int k) {
    return (k == 0 || k == 5) ? 64.f : ((k == 1 || k == 3 || k == 6) ? 16.f : 4.f);
  }
};

template <> struct Unpacker<2, true> {
  static constexpr int NP = 8;
  uint32_t m01, m23, m45, m67, m89, e1024, e256, e64, e16, e4;
  __device__ __forceinline__ Unpacker()
      : m01(opaque_sgpr(0x00030003u)), m23(opaque_sgpr(0x000C000Cu)), m45(opaque_sgpr(0x00300030u)),
        m67(opaque_sgpr(0x00C000C0u)), m89(opaque_sgpr(0x03000300u)),
        e1024(opaque_vgpr(0x64006400u)), e256(opaque_vgpr(0x5C005C00u)), e64(opaque_vgpr(0x54005400u)),
        e16(opaque_vgpr(0x4C004C00u)), e4(opaque_vgpr(0x44004400u)) {}
  __device__ __forceinline__ void run(uint32_t w, uint32_t* v) const {
    const uint32_t c = w >> 6;
    v[0] = and_or(w, m01, e1024);  // mantissa bits 0-1: 1024 + code
    v[1] = and_or(w, m23, e256);   // bits 2-3: 256 + code
    v[2] = and_or(w, m45, e64);
    v[3] = and_or(w, m67, e16);
    v[4] = and_or(w, m89, e4);
    v[5] = and_or(c, m45, e64);
    v[6] = and_or(c, m67, e16);
    v[7] = and_or(c, m89, e4);
  }
  __device__ static __forceinline__ float offset(int k) {
    return k == 0 ? 1024.f : k == 1 ? 256.f : (k == 2 || k == 5) ? 64.f : (k == 3 || k == 6) ? 16.f : 4.f;
  }
};

template <> struct Unpacker<4, false> {
  static constexpr int NP = 4;
  uint32_t m, e64;
  __device__ __forceinline__ Unpacker() : m(opaque_sgpr(0x00F000F0u)), e64(opaque_vgpr(0x54005400u)) {}
  __device__ __forceinline__ void run(uint32_t w, uint32_t* v) const {
    v[0] = and_or(w << 4, m, e64);   // mantissa bits 4-7: 64 + code
    v[1] = and_or(w, m, e64);
    v[2] = and_or(w >> 4, m, e64);
    v[3] = and_or(w >> 8, m, e64);
  }
  __device__ static __forceinline__ float offset(int) { return 64.f; }
};

template <> struct Unpacker<4, true> {
  static constexpr int NP = 4;
  uint32_t m03, m47, e1024, e64;
  __device__ __forceinline__ Unpacker()
      : m03(opaque_sgpr(0x000F000Fu)), m47(opaque_sgpr(0x00F000F0u)),
        e1024(opaque_vgpr(0x64006400u)), e64(opaque_vgpr(0x54005400u)) {}
  __device__ __forceinline__ void run(uint32_t w, uint32_t* v) const {
    v[0] = and_or(w, m03, e1024);        // mantissa bits 0-3: 1024 + code
    v[1] = and_or(w, m47, e64);          // bits 4-7: 64 + code
    v[2] = and_or(w >> 4, m47, e64);
    v[3] = and_or(w >> 12, m03, e1024);
  }
  __device__ static __forceinline__ float offset(int k) { return (k == 0 || k == 3) ? 1024.f : 64.f; }
};

template <bool WIDE> struct Unpacker<8, WIDE> {
  static constexpr int NP = 2;
  uint32_t m, e1024;
  __device__ __forceinline__ Unpacker() : m(opaque_sgpr(0x00FF00FFu)), e1024(opaque_vgpr(0x64006400u)) {}
  __device__ __forceinline__ void run(uint32_t w, uint32_t* v) const {
    v[0] = and_or(w, m, e1024);          // mantissa bits 0-7: 1024 + code
    v[1] = and_or(w >> 8, m, e1024);
  }
  __device__ static __forceinline__ float offset(int) { return 1024.f; }
};

// ---------------------------------------------------------------------------
// Cross-lane reductions of a wave64 (DPP within rows of 16 lanes, permlane
// swaps across rows; no LDS).
__device__ __forceinline__ uint32_t fbits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float bitsf(uint32_t x) { return __builtin_bit_cast(float, x); }

// v + rotate_right(v, s) within each row of 16 lanes.
template <int S>
__device__ __forceinline__ float row_ror_add(float v) {
  return v + __builtin_amdgcn_update_dpp(0.f, v, 0x120 + S, 0xF, 0xF, false);
}

// Sum over aligned groups of N consecutive lanes (N = 1, 2, 4, 8, 16) with
// DPP: quad permutations, then half-row and row mirrors.  Every lane of a
// group ends with the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if (N >= 2) x += __builtin_amdgcn_update_dpp(0.f, x, 0xB1, 0xF, 0xF, false);   // [1,0,3,2]
  if (N >= 4) x += __builtin_amdgcn_update_dpp(0.f, x, 0x4E, 0xF, 0xF, false);   // [2,3,0,1]
  if (N >= 8) x += __builtin_amdgcn_update_dpp(0.f, x, 0x141, 0xF, 0xF, false);  // half mirror
  if (N >= 16) x += __builtin_amdgcn_update_dpp(0.f, x, 0x140, 0xF, 0xF, false); // mirror
  return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x) {
  if (N >= 2) x = fmaxf(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false));
  if (N >= 4) x = fmaxf(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false));
  if (N >= 8) x = fmaxf(x, __builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false));
  if (N >= 16) x = fmaxf(x, __builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false));
  return x;
}

// For x uniform within each row of 16 lanes: the sum over row pairs (0,1) and
// (2,3) [ROWS == 2] or over all four rows [ROWS == 4], in every lane.
template <int ROWS>
__device__ __forceinline__ float xrow_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(fbits(x), fbits(x), false, false);
  x = bitsf(a[0]) + bitsf(a[1]);
  if (ROWS == 4) {
    const auto b = __builtin_amdgcn_permlane32_swap(fbits(x), fbits(x), false, false);
    x = bitsf(b[0]) + bitsf(b[1]);
  }
  return x;
}

__device__ __forceinline__ float wave_sum64(float x) { return xrow_sum<4>(group_sum<16>(x)); }

__device__ __forceinline__ float wave_max64(float x) {
  x = group_max<16>(x);
  const auto a = __builtin_amdgcn_permlane16_swap(fbits(x), fbits(x), false, false);
  x = fmaxf(bitsf(a[0]), bitsf(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(fbits(x), fbits(x), false, false);
  return fmaxf(bitsf(b[0]), bitsf(b[1]));
}


// Bitwise OR over aligned groups of N consecutive lanes (N = 1, 2, 4, 8, 16).
template <int N>
__device__ __forceinline__ uint32_t group_or(uint32_t x) {
  if (N >= 2) x |= __builtin_amdgcn_update_dpp(0u, x, 0xB1, 0xF, 0xF, false);
  if (N >= 4) x |= __builtin_amdgcn_update_dpp(0u, x, 0x4E, 0xF, 0xF, false);
  if (N >= 8) x |= __builtin_amdgcn_update_dpp(0u, x, 0x141, 0xF, 0xF, false);
  if (N >= 16) x |= __builtin_amdgcn_update_dpp(0u, x, 0x140, 0xF, 0xF, false);
  return x;
}

template <int N>
__device__ __forceinline__ float group_min(float x) {
  if (N >= 2) x = fminf(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false));
  if (N >= 4) x = fminf(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false));
  if (N >= 8) x = fminf(x, __builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false));
  if (N >= 16) x = fminf(x, __builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false));
  return x;
}

// min / max over aligned groups of N lanes, N = 16, 32 or 64 (every lane of
// a group gets the group's value).
template <int N>
__device__ __forceinline__ float span_min(float x) {
  x = group_min<16>(x);
  if (N >= 32) {
    const auto a = __builtin_amdgcn_permlane16_swap(fbits(x), fbits(x), false, false);
    x = fminf(bitsf(a[0]), bitsf(a[1]));
  }
  if (N >= 64) {
    const auto b = __builtin_amdgcn_permlane32_swap(fbits(x), fbits(x), false, false);
    x = fminf(bitsf(b[0]), bitsf(b[1]));
  }
  return x;
}
template <int N>
__device__ __forceinline__ float span_max(float x) {
  x = group_max<16>(x);
  if (N >= 32) {
    const auto a = __builtin_amdgcn_permlane16_swap(fbits(x), fbits(x), false, false);
    x = fmaxf(bitsf(a[0]), bitsf(a[1]));
  }
  if (N >= 64) {
    const auto b = __builtin_amdgcn_permlane32_swap(fbits(x), fbits(x), false, false);
    x = fmaxf(bitsf(b[0]), bitsf(b[1]));
  }
  return x;
}

}  // namespace kvq
