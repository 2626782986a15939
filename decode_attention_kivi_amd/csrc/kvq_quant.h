// Quantizer pieces shared by the quantize kernels and the decode kernel's
// fused append: one group's fp16 scale / zero point and the codes, and one
// stream's decode-step append.
//
// Bit-exact contract (include/kvq.h): every step is one IEEE fp32 operation
// on fp16-exact inputs -- subtract, correctly rounded divide, round half to
// even -- with no FMA contraction, in every file that includes this one.
// The divide is only needed where it can change the code: see encode().
#pragma once

#include "kvq_internal.h"
#include "kvq_device.h"

namespace kvq {

// One group's scale and zero point.  Zero extrema are canonicalized to +0
// (min/max of {-0, +0} are not ordered), so z and s have single encodings.
struct GroupScale {
  uint32_t s16, z16;
  float s, z;
  float inv;              // v_rcp_f32(s), within 1 ulp of 1/s; 0 when s == 0 (all codes 0)
};

// fl(D / qmax) for qmax = 3, 15 or 255 without a division: q0 = fl(D c) with
// c = fl(1/qmax), the residual r = D - q0 qmax (exact, one fma) and
// fl(q0 + r c).  Equal to the correctly rounded quotient for every fp32 D in
// [2^-24, 2^17) (tried exhaustively, one binade at a time, on the host: the
// steps scale exactly with D's exponent there), 0 for D = 0 and +inf for
// D = +inf (an infinite input; the residual would be NaN).
template <int BITS>
__device__ __forceinline__ float div_qmax(float D) {
  constexpr float kQmax = float((1 << BITS) - 1);
  constexpr float kInv = 1.0f / kQmax;
  const float q0 = D * kInv;
  const float r = __builtin_fmaf(-q0, kQmax, D);
  const float q = __builtin_fmaf(r, kInv, q0);
  return q0 == __builtin_inff() ? q0 : q;
}

template <int BITS>
__device__ __forceinline__ GroupScale group_scale(float mn, float mx) {
#pragma clang fp contract(off)
  GroupScale g;
  mn = mn + 0.0f;
  mx = mx + 0.0f;
  g.s16 = f2h(div_qmax<BITS>(mx - mn));   // mn, mx fp16 values: mx - mn is 0 or in [2^-24, 131008]
  g.z16 = f2h(mn);
  g.s = h2f(g.s16);
  g.z = mn;                  // mn is an fp16 value: z16 holds it exactly
  g.inv = g.s == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(g.s);
  return g;
}

// code = clamp(rint(fl(d / s))), d = fl(x - z), with fl(d / s) the correctly
// rounded quotient (the definition).
template <int BITS>
__device__ __forceinline__ uint32_t encode(float x, const GroupScale& g) {
#pragma clang fp contract(off)
  constexpr float kQmax = float((1 << BITS) - 1);
  if (g.s == 0.0f) return 0u;
  float t = rintf(__fdiv_rn(x - g.z, g.s));
  t = fminf(fmaxf(t, 0.0f), kQmax);
  return static_cast<uint32_t>(t);
}

// The same code without the division where it cannot matter: q = fl(d * inv)
// lies within |d/s| * 2^-22 of the correctly rounded quotient (inv within
// 2^-23 relative of 1/s, two roundings of 2^-24), so rint gives the same
// integer for both unless a half-integer lies that close to q.  Inside a
// group |d/s| <= 1.5 (2^b - 1) (d <= max - min; s is (max - min)/(2^b - 1)
// rounded to fp16, low by at most a factor 1.5 in the subnormal range), so
// `near` is set when q is within 2^b 2^-20 -- over 2.6 times the largest
// bound -- of a half-integer; the caller then encodes again with encode(),
// for the whole wave (one uniform branch per batch of elements).  q - rint(q)
// is exact.  s == 0 has inv = 0: q = 0, code 0, never near.
template <int BITS>
__device__ __forceinline__ uint32_t encode_fast(float x, const GroupScale& g, bool& near) {
#pragma clang fp contract(off)
  constexpr float kQmax = float((1 << BITS) - 1);
  constexpr float kFar = 0.5f - float(1 << BITS) * 0x1p-20f;   // exact
  const float q = (x - g.z) * g.inv;
  const float t = rintf(q);
  near |= fabsf(q - t) >= kFar;
  return static_cast<uint32_t>(fminf(fmaxf(t, 0.0f), kQmax));
}

// true on every lane when any lane of the wave sets x
__device__ __forceinline__ bool wave_any(bool x) { return __builtin_amdgcn_ballot_w64(x) != 0; }

// ---------------------------------------------------------------------------
// Row-batch encoder of the wave quantizers: 8 channels held as fp16 pairs
// (channel 2e in the low half of word e of a 16-byte row piece).

// Packed fp16 min / max (v_pk_min_f16 / v_pk_max_f16, both halves at once).
// Exact; the sign of a zero result is not specified, which group_scale's
// canonicalization makes irrelevant.
__device__ __forceinline__ uint32_t pk_min_f16(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_min_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ uint32_t pk_max_f16(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_max_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// fl(x - z) for x the fp16 in the low (HI false) or high half of w, in one
// v_fma_mix_f32: x widened exactly, times one (1.0, held in a scalar
// register), plus -z (the source negate modifier), one rounding -- the same
// value as converting x and subtracting in fp32.
template <bool HI>
__device__ __forceinline__ float sub_half_f32(uint32_t w, float one, float z) {
  float r;
  if constexpr (HI)
    asm("v_fma_mix_f32 %0, %1, %2, -%3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "s"(one), "v"(z));
  else
    asm("v_fma_mix_f32 %0, %1, %2, -%3 op_sel:[0,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "s"(one), "v"(z));
  return r;
}

// A group whose scale lets the reciprocal path skip the clamp: s = 0 (inv 0,
// every code 0) or s a normal finite fp16.  Then z = min exactly (the extrema
// are fp16 values), so d = fl(x - z) >= 0, and with s >= (1 - 2^-11)
// fl(max - min)/(2^b - 1) the product q stays below (2^b - 1)(1 + 2^-10)
// < 2^b - 1/2: rint(q) is a code without clamping.  Subnormal scales (rounded
// by up to a factor 1.5) and infinite ones go through encode().
__device__ __forceinline__ bool scale_unclamped(uint32_t s16) {
  return s16 == 0u || (s16 >= 0x0400u && s16 < 0x7C00u);
}

// Codes of the 8 channels of x, by the reciprocal product and without the
// clamp (valid for scale_unclamped groups), packed as 16-bit chunks of
// 16/BITS codes (channel c at bits BITS*(c % (16/BITS)) of chunk
// c / (16/BITS)).  Each code goes into its chunk by one exact fp32 fma
// (integers below 2^16).  err collects |q - rint(q)|; a batch with
// err >= 1/2 - 2^b 2^-20 anywhere in the wave is encoded again by encode()
// (see encode_fast for the bound).  z[c], inv[c] of channel c's group.
template <int BITS>
__device__ __forceinline__ void codes8_fast(const uint4& x, const float (&z)[8], const float (&inv)[8],
                                            float one, float& err, uint32_t (&chunk)[BITS / 2]) {
#pragma clang fp contract(off)
  constexpr int KPC = 16 / BITS;         // codes per 16-bit chunk
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  float acc[BITS / 2];
  float r[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float d = (c & 1) ? sub_half_f32<true>(w[c / 2], one, z[c]) : sub_half_f32<false>(w[c / 2], one, z[c]);
    const float q = d * inv[c];
    const float t = rintf(q);
    r[c] = q - t;
    const int j = c % KPC;
    if (j == 0) acc[c / KPC] = t;
    else acc[c / KPC] = __builtin_fmaf(t, float(1 << (BITS * j)), acc[c / KPC]);
  }
#pragma unroll
  for (int c = 0; c < 8; c += 2) err = fmaxf(err, fmaxf(fabsf(r[c]), fabsf(r[c + 1])));
#pragma unroll
  for (int m = 0; m < BITS / 2; ++m) chunk[m] = static_cast<uint32_t>(acc[m]);
}

// The same chunks from the definition (encode(): correctly rounded quotient,
// clamp) -- the path of batches the fast one cannot decide.
template <int BITS>
__device__ __forceinline__ void codes8_exact(const uint4& x, const GroupScale (&g)[8], uint32_t (&chunk)[BITS / 2]) {
  constexpr int KPC = 16 / BITS;
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int m = 0; m < BITS / 2; ++m) chunk[m] = 0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float f = h2f((c & 1) ? (w[c / 2] >> 16) : (w[c / 2] & 0xffffu));
    chunk[c / KPC] |= encode<BITS>(f, g[c]) << (BITS * (c % KPC));
  }
}

// Bound of the reciprocal path: |q - rint(q)| at or above it may round
// differently from the correctly rounded quotient.
template <int BITS>
constexpr float kFastFar = 0.5f - float(1 << BITS) * 0x1p-20f;

// One decode step's append for stream s, by one wave (KIVI note, Algorithm 1,
// Decoding): lanes 0..D/8-1 copy the new key row into key-residual row
// k_row, lanes D/8..D/4-1 the new value row into value-window row v_row (16
// bytes per lane); then, when v_quant_row >= 0, the window row v_quant_row
// (the new row itself when it is v_row) is quantized per token with each
// lane holding D/64 channels: group min/max by cross-lane reductions, codes
// from group_scale / encode, 16-bit units assembled by OR across the lanes of
// a unit, written as token v_dst_tok of the value run with its (scale, zero)
// pairs (at an even token the pair partner's halves and pairs are zeroed).
template <int BITS, int D, int G>
__device__ __forceinline__ void append_stream(const AppendParams& p, int64_t s, int lane) {
#pragma clang fp contract(off)

  constexpr int CPL = D / 64;            // channels per lane
  constexpr int LPG = G / CPL;           // lanes per group: 16, 32 or 64
  constexpr int NG = D / G;
  constexpr int KPU = 16 / BITS;         // codes per 16-bit unit
  constexpr int LPU = KPU / CPL;         // lanes per unit
  if (lane < D / 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(p.k_new + s * p.k_new_stride + lane * 8);
    *reinterpret_cast<uint4*>(p.k_res + s * p.k_res_stride + int64_t(p.k_row) * D + lane * 8) = v;
  } else if (lane < D / 4) {
    const int c = lane - D / 8;
    const uint4 v = *reinterpret_cast<const uint4*>(p.v_new + s * p.v_new_stride + c * 8);
    *reinterpret_cast<uint4*>(p.v_res + s * p.v_res_stride + int64_t(p.v_row) * D + c * 8) = v;
  }
  if (p.v_quant_row < 0) return;
  // the row being quantized is read where it is complete: the new value
  // itself if it is the row written in this launch
  const uint16_t* row = p.v_quant_row == p.v_row
                            ? p.v_new + s * p.v_new_stride
                            : p.v_res + s * p.v_res_stride + int64_t(p.v_quant_row) * D;
  float xv[CPL];
  if constexpr (CPL == 2) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(row)[lane];
    xv[0] = h2f(w & 0xffffu);
    xv[1] = h2f(w >> 16);
  } else {
    xv[0] = h2f(row[lane]);
  }
  float mn = xv[0], mx = xv[0];
  if constexpr (CPL == 2) {
    mn = fminf(mn, xv[1]);
    mx = fmaxf(mx, xv[1]);
  }
  mn = span_min<LPG>(mn);
  mx = span_max<LPG>(mx);
  const GroupScale gs = group_scale<BITS>(mn, mx);
  uint32_t unit = 0;
  bool near = false;
#pragma unroll
  for (int k = 0; k < CPL; ++k) unit |= encode_fast<BITS>(xv[k], gs, near) << (((lane * CPL + k) % KPU) * BITS);
  if (wave_any(near)) {
    unit = 0;
#pragma unroll
    for (int k = 0; k < CPL; ++k) unit |= encode<BITS>(xv[k], gs) << (((lane * CPL + k) % KPU) * BITS);
  }
  unit = group_or<LPU>(unit);
  const int64_t te = p.v_dst_tok;
  const int64_t pair = te >> 1;
  const int par = int(te & 1);
  constexpr int64_t rb = int64_t(D) * BITS / 8;
  uint8_t* blk = p.v_codes + s * p.v_codes_stride + pair * 2 * rb;
  uint32_t* meta = reinterpret_cast<uint32_t*>(p.v_meta + s * p.v_meta_stride);
  const int uidx = lane * CPL / KPU;     // unit of the row = word of the pair block
  const int g = lane / LPG;
  if (lane % LPU == 0) {
    *reinterpret_cast<uint16_t*>(blk + 4 * uidx + 2 * par) = static_cast<uint16_t>(unit);
    if (par == 0) *reinterpret_cast<uint16_t*>(blk + 4 * uidx + 2) = 0;   // unwritten partner
  }
  if (lane % LPG == 0) {
    meta[(pair * NG + g) * 2 + par] = gs.s16 | (gs.z16 << 16);
    if (par == 0) meta[(pair * NG + g) * 2 + 1] = 0u;
  }
}

}  // namespace kvq
