// Decode-step attention over a low-bit quantized KV cache, split over the
// context (the FlashDecoding dataflow that the VQ-LLM note's reference [10]
// describes) with a final cross-split softmax merge.
//
// A workgroup takes one cache stream (batch b, kv head h), the GQ query heads
// that share it, and a range of tokens whose keys come from one source (a
// quantized run or the fp16 residual) and whose values come from one source.
// Each of its four waves streams its own sub-range independently; the only
// workgroup barrier is the final combine.  Per wave:
//   1. q*s for every key group of the range (per-channel key scales, KIVI
//      note "Method details"), as fp16 hi + lo pairs, and the group bias
//      sum_c q_c z_c, into the wave's LDS area;
//   2. logits: prefetched 16-byte loads of packed codes, unpack of code pairs
//      into fp16 (offset + code) by mask-and-or with an exponent constant,
//      v_dot2_f32_f16 against q*s; residual rows dot q directly
//      (A = Concat([A_g, A_r]));
//   3. the range's max and sum of exp2(logit - max): one softmax over the
//      concatenation (KIVI Algorithm 1; WindowQuant Sec. 3.3.1);
//   4. A.V over token-pair value blocks: one fp16 pair holds the same channel
//      of two tokens, so v_dot2 applies both tokens' p*s at once; sum(p*z) and
//      sum(p*s) per group are kept apart and folded in at the end; partials
//      are reduced with DPP row rotations and a 4-row LDS stage;
//   5. the four waves' (max, sum, o[d]) are combined and written as the
//      split's partial; the merge kernel rescales and adds the splits.
// Logits are kept in base 2 (q is pre-scaled by sm_scale * log2 e).

#include "kvq_internal.h"
#include "kvq_device.h"

namespace kvq {
namespace {

constexpr int NT = kThreads;
constexpr int NB = 8;    // loads per batch in the key streaming loops (wave instructions)
constexpr int NBV = 4;   // loads per batch in the value streaming loops

// Make this wave's LDS writes visible to its own later LDS reads.  LDS
// operations of one wave execute in order; this only keeps the compiler from
// moving memory operations across the point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// v + rotate_right(v, s) within each row of 16 lanes.
template <int S>
__device__ __forceinline__ float row_ror_add(float v) {
  return v + __builtin_amdgcn_update_dpp(0.f, v, 0x120 + S, 0xF, 0xF, false);
}

// Sum over aligned groups of N consecutive lanes (N = 1, 2, 4, 8, 16) with
// DPP: quad permutations, then half-row and row mirrors.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if (N >= 2) x += __builtin_amdgcn_update_dpp(0.f, x, 0xB1, 0xF, 0xF, false);   // [1,0,3,2]
  if (N >= 4) x += __builtin_amdgcn_update_dpp(0.f, x, 0x4E, 0xF, 0xF, false);   // [2,3,0,1]
  if (N >= 8) x += __builtin_amdgcn_update_dpp(0.f, x, 0x141, 0xF, 0xF, false);  // half mirror
  if (N >= 16) x += __builtin_amdgcn_update_dpp(0.f, x, 0x140, 0xF, 0xF, false); // mirror
  return x;
}

struct WaveLds {
  float* logit;      // [GQ][LT] logits by token slot; later the [4][D] value rows
  uint16_t* p16;     // [GQ][LT] fp16 probabilities, zero outside the wave's tokens
  uint32_t* qs;      // [NGW][GQ][2][D/2] q*s fp16 hi pairs then lo pairs
  float* bias;       // [NGW][GQ]
  float* ow;         // [GQ][D+2] (m, l, o[D]) of the wave (aliases qs/bias)
};

template <int D, int GQ>
__device__ __forceinline__ WaveLds carve_wave(unsigned char* smem, int wave) {
  constexpr int NGW = wave_tokens(GQ) / 32 + 1;
  constexpr DecodeLds lay = decode_lds(D, GQ);
  unsigned char* base = smem + lay.block + int64_t(wave) * lay.wave;
  WaveLds W;
  W.logit = reinterpret_cast<float*>(base);
  W.p16 = reinterpret_cast<uint16_t*>(base + lay.logit);
  W.qs = reinterpret_cast<uint32_t*>(base + lay.logit + lay.p16);
  W.bias = reinterpret_cast<float*>(base + lay.logit + lay.p16 + int64_t(NGW) * GQ * D * 4);
  W.ow = reinterpret_cast<float*>(base + lay.logit + lay.p16);
  return W;
}

__device__ __forceinline__ half2_t as_h2(uint32_t x) { return __builtin_bit_cast(half2_t, x); }
__device__ __forceinline__ uint32_t as_u32(half2_t x) { return __builtin_bit_cast(uint32_t, x); }

// ---------------------------------------------------------------------------
// Keys of run tokens [r0, r1) (bits 2/4/8) -> logits at slots slot0 + (t - r0).
//
// Per key group: hi = fp16(q'*s), lo = fp16(q'*s - hi) with packed fp16 ops
// (q' = q * 2^-8 exactly, so no product can overflow fp16); a single fp16
// q*s is too coarse for outlier channels, whose large logits would carry its
// 2^-11 relative error into the softmax, while hi + lo keeps ~22 bits.  The
// bias sum_c q'_c z_c - sum_c (hi + lo)_c * offset_c comes from three dot2.
template <int D, int GQ, int BITS>
__device__ void keys_quantized(const DecodeParams& P, const WaveLds& W, const uint16_t* qh16,
                               int64_t stream, const Run& run, int r0, int r1, int slot0,
                               int lane) {
  constexpr int LT = wave_tokens(GQ) + 4;
  constexpr int RB = D * BITS / 8;       // bytes per token row
  constexpr int CPR = RB / 16;           // 16-byte chunks per row
  constexpr int TPI = 64 / CPR;          // tokens per wave instruction
  constexpr int PPC = 64 / BITS;         // fp16 pairs per chunk
  constexpr int NP = Unpack<BITS>::NP;   // pairs per 32-bit word
  constexpr int CPW = 32 / BITS;         // channels per 32-bit word
  constexpr int HD = D / 2;              // pairs per row
  constexpr int GPI = 64 / HD;           // key groups per meta iteration
  constexpr int NGW = wave_tokens(GQ) / 32 + 1;
  constexpr int MI = (NGW + GPI - 1) / GPI;
  const int lg = P.lg_g;
  const int j0 = r0 >> lg;
  const int ng = ((r1 - 1) >> lg) - j0 + 1;
  const int rofs = r0 & (P.G - 1);
  const int n = r1 - r0;
  const uint8_t* codes = P.k_codes + stream * P.k_codes_stride + run.code_off;
  const uint32_t* meta = reinterpret_cast<const uint32_t*>(
      P.k_meta + stream * P.k_meta_stride + run.meta_off);
  const int n_inst = (n + TPI - 1) / TPI;
  const int my_t = lane / CPR, my_c = lane % CPR;

  // the first batch of code loads is in flight during the meta work; every
  // load address is clamped into the range, so no load sits behind a branch
  auto load = [&](int i) {
    const int r = r0 + min(i * TPI + my_t, n - 1);
    return *reinterpret_cast<const uint4*>(codes + int64_t(r) * RB + my_c * 16);
  };
  uint4 buf[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) buf[u] = load(u);

  // meta work: lane -> pair pi of a row (word pi/NP, position pi%NP, i.e.
  // channels clo and clo + NP) of group it*GPI + lane/HD
  const int pi = lane % HD, gsub = lane / HD;
  const int kq = pi % NP;
  const int clo = (pi / NP) * CPW + kq, chi = clo + NP;
  uint32_t mlo[MI], mhi[MI];
#pragma unroll
  for (int it = 0; it < MI; ++it) {
    const int j = min(it * GPI + gsub, ng - 1);
    const uint32_t* m = meta + int64_t(j0 + j) * D;
    mlo[it] = m[clo];
    mhi[it] = m[chi];
  }
  half2_t qk[GQ];
#pragma unroll
  for (int h = 0; h < GQ; ++h)
    qk[h] = as_h2(uint32_t(qh16[h * D + clo]) | (uint32_t(qh16[h * D + chi]) << 16)) *
            as_h2(0x1C001C00u);                                   // * 2^-8, exact
  const _Float16 off = static_cast<_Float16>(Unpack<BITS>::offset(kq));
  const half2_t nego = {-off, -off};
#pragma unroll
  for (int it = 0; it < MI; ++it) {
    const int j = it * GPI + gsub;
    const bool valid = j < ng;
    if (it * GPI >= ng) continue;          // uniform; keeps the loop fully unrolled
    const half2_t s2 = as_h2((mlo[it] & 0xffffu) | (mhi[it] << 16));
    const half2_t z2 = as_h2((mlo[it] >> 16) | (mhi[it] & 0xffff0000u));
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      const half2_t hi = qk[h] * s2;
      const half2_t lo = __builtin_elementwise_fma(qk[h], s2, -hi);
      float bp = __builtin_amdgcn_fdot2(qk[h], z2, 0.f, false);
      bp = __builtin_amdgcn_fdot2(hi, nego, bp, false);
      bp = __builtin_amdgcn_fdot2(lo, nego, bp, false);
      bp = group_sum<16>(bp);
      bp += __shfl_xor(bp, 16);
      if (HD == 64) bp += __shfl_xor(bp, 32);
      if (valid) {
        uint32_t* qs = W.qs + (j * GQ + h) * (2 * HD);
        qs[pi] = as_u32(hi);
        qs[HD + pi] = as_u32(lo);
        if (pi == 0) W.bias[j * GQ + h] = bp;
      }
    }
  }
  wave_lds_sync();

  const float sc = P.scale_log2 * 256.f;   // undo the 2^-8
  for (int i0 = 0;;) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int i = i0 + u;
      const uint4 cw = buf[u];
      const int tl = i * TPI + my_t;
      const bool valid = tl < n;
      const int jl = (min(tl, n - 1) + rofs) >> lg;
      uint32_t v[4][NP];
      Unpack<BITS>::run(cw.x, v[0]);
      Unpack<BITS>::run(cw.y, v[1]);
      Unpack<BITS>::run(cw.z, v[2]);
      Unpack<BITS>::run(cw.w, v[3]);
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        const uint32_t* qb = W.qs + (jl * GQ + h) * (2 * HD) + my_c * PPC;
        const uint4* qhi = reinterpret_cast<const uint4*>(qb);
        const uint4* qlo = reinterpret_cast<const uint4*>(qb + HD);
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
#pragma unroll
          for (int q4 = 0; q4 < NP / 4 + (NP < 4 ? 1 : 0); ++q4) {
            const int pbase = w * NP + q4 * 4;   // the NP pairs of word w
            uint32_t hi[4], lo[4];
            if (NP >= 4) {
              const uint4 x = qhi[pbase / 4], y = qlo[pbase / 4];
              hi[0] = x.x; hi[1] = x.y; hi[2] = x.z; hi[3] = x.w;
              lo[0] = y.x; lo[1] = y.y; lo[2] = y.z; lo[3] = y.w;
            } else {
              const uint2 x = reinterpret_cast<const uint2*>(qb)[pbase / 2];
              const uint2 y = reinterpret_cast<const uint2*>(qb + HD)[pbase / 2];
              hi[0] = x.x; hi[1] = x.y; lo[0] = y.x; lo[1] = y.y;
            }
#pragma unroll
            for (int e = 0; e < (NP >= 4 ? 4 : NP); ++e) {
              acc = dot2(hi[e], v[w][q4 * 4 + e], acc);
              acc = dot2(lo[e], v[w][q4 * 4 + e], acc);
            }
          }
        }
        acc = group_sum<CPR>(acc);
        if (valid && my_c == 0) W.logit[h * LT + slot0 + tl] = (acc + W.bias[jl * GQ + h]) * sc;
      }
    }
    i0 += NB;
    if (i0 >= n_inst) break;
    // the whole batch is consumed before the next one is issued, so no load
    // is in flight across the loop edge and the wait counts stay exact
#pragma unroll
    for (int u = 0; u < NB; ++u) buf[u] = load(i0 + u);
  }
}

// Keys from fp16 rows rows[row0 + i], i < n -> logits at slots slot0 + i.
template <int D, int GQ>
__device__ void keys_fp16(const DecodeParams& P, const WaveLds& W, const uint16_t* qh16,
                          const uint16_t* rows, int row0, int n, int slot0, int lane) {
  constexpr int LT = wave_tokens(GQ) + 4;
  constexpr int CPR = D / 8;             // 16-byte chunks per row
  constexpr int TPI = 64 / CPR;
  const int n_inst = (n + TPI - 1) / TPI;
  const int my_t = lane / CPR, my_c = lane % CPR;
  auto load = [&](int i) {
    const int t = min(i * TPI + my_t, n - 1);
    return *reinterpret_cast<const uint4*>(rows + int64_t(row0 + t) * D + my_c * 8);
  };
  uint4 buf[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) buf[u] = load(u);
  for (int i0 = 0;;) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int i = i0 + u;
      const uint4 x = buf[u];
      const int t = i * TPI + my_t;
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        const uint4 qq = reinterpret_cast<const uint4*>(qh16 + h * D)[my_c];
        float acc = dot2(qq.x, x.x, 0.f);
        acc = dot2(qq.y, x.y, acc);
        acc = dot2(qq.z, x.z, acc);
        acc = dot2(qq.w, x.w, acc);
        acc = group_sum<CPR>(acc);
        if (t < n && my_c == 0) W.logit[h * LT + slot0 + t] = acc * P.scale_log2;
      }
    }
    i0 += NB;
    if (i0 >= n_inst) break;
#pragma unroll
    for (int u = 0; u < NB; ++u) buf[u] = load(i0 + u);
  }
}

// ---------------------------------------------------------------------------
// Reduce the per-lane value partials vals[CH] (lanes l with l % CPL == c own
// channels c*CH .. c*CH+CH-1) across the wave into o[0..D).  The four rows of
// 16 lanes are combined through W.logit, whose logits are dead by now.
template <int D, int CPL, int CH>
__device__ __forceinline__ void wave_reduce_values(const WaveLds& W, float* vals, int lane,
                                                   float* o) {
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    float x = vals[j];
    if (CPL <= 8) x = row_ror_add<8>(x);
    if (CPL <= 4) x = row_ror_add<4>(x);
    if (CPL <= 2) x = row_ror_add<2>(x);
    if (CPL <= 1) x = row_ror_add<1>(x);
    vals[j] = x;
  }
  // lanes (lane % 16) < CPL of each row of 16 now hold their row's sums
  float* red = W.logit;
  const int row = lane >> 4, c = lane & 15;
  if (c < CPL) {
#pragma unroll
    for (int j = 0; j < CH; ++j) red[row * D + c * CH + j] = vals[j];
  }
  wave_lds_sync();
  for (int ch = lane; ch < D; ch += 64)
    o[ch] = (red[ch] + red[D + ch]) + (red[2 * D + ch] + red[3 * D + ch]);
  wave_lds_sync();
}

// Values of run tokens [r0, r1) (bits 2/4/8).  Pair block P of the run holds
// run tokens 2P and 2P+1, whose probabilities are the fp16 pair P - r0/2 of
// W.p16 (slot 2(P - r0/2) is token 2P); the pair after the last is zero.
template <int D, int GQ, int BITS>
__device__ void values_quantized(const DecodeParams& P, const WaveLds& W, int64_t stream,
                                 const Run& run, int r0, int r1, int lane) {
  constexpr int LT = wave_tokens(GQ) + 4;
  constexpr int RB = D * BITS / 8;
  constexpr int CPP = 2 * RB / 16;        // 16-byte chunks per pair block
  constexpr int PPI = 64 / CPP;           // pair blocks per wave instruction
  constexpr int CPCV = 64 / BITS;         // channels per chunk
  constexpr int NP = Unpack<BITS>::NP;    // channels per 16-bit unit
  constexpr int HPP = (GQ * CPCV <= 64) ? GQ : ((64 / CPCV) > 0 ? (64 / CPCV) : 1);
  const int NG = D >> P.lg_g;
  const int my_p = lane / CPP, my_c = lane % CPP;
  const int g = (my_c * CPCV) >> P.lg_g;
  const int p0 = r0 >> 1;
  const int np = ((r1 - 1) >> 1) - p0 + 1;
  const int n_inst = (np + PPI - 1) / PPI;
  const uint8_t* codes = P.v_codes + stream * P.v_codes_stride + run.code_off;
  const uint8_t* meta = P.v_meta + stream * P.v_meta_stride + run.meta_off;
  const uint32_t* pp = reinterpret_cast<const uint32_t*>(W.p16);
  const half2_t one2 = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};

  for (int hp = 0; hp < GQ; hp += HPP) {
    float acc[HPP][CPCV];
    float sps[HPP], pz[HPP];
#pragma unroll
    for (int hh = 0; hh < HPP; ++hh) {
      sps[hh] = 0.f;
      pz[hh] = 0.f;
#pragma unroll
      for (int j = 0; j < CPCV; ++j) acc[hh][j] = 0.f;
    }
    auto load = [&](int i, uint4& c4, uint2& m2) {
      const int64_t pr = p0 + min(i * PPI + my_p, np - 1);
      c4 = *reinterpret_cast<const uint4*>(codes + pr * (2 * RB) + my_c * 16);
      m2 = *reinterpret_cast<const uint2*>(meta + (pr * NG + g) * 8);
    };
    uint4 cb[NBV];
    uint2 mb[NBV];
#pragma unroll
    for (int u = 0; u < NBV; ++u) load(u, cb[u], mb[u]);
    for (int i0 = 0;;) {
#pragma unroll
      for (int u = 0; u < NBV; ++u) {
        const int i = i0 + u;
        const uint4 cw = cb[u];
        const uint2 mw = mb[u];
        const int plc = min(i * PPI + my_p, np);      // pair np reads as zero
        const half2_t s2 = as_h2((mw.x & 0xffffu) | (mw.y << 16));
        const half2_t z2 = as_h2((mw.x >> 16) | (mw.y & 0xffff0000u));
        uint32_t ps[HPP];
#pragma unroll
        for (int hh = 0; hh < HPP; ++hh) {
          const half2_t p2 = as_h2(pp[(hp + hh) * (LT / 2) + plc]);
          const half2_t psh = p2 * s2;
          ps[hh] = as_u32(psh);
          sps[hh] = __builtin_amdgcn_fdot2(psh, one2, sps[hh], false);
          pz[hh] = __builtin_amdgcn_fdot2(p2, z2, pz[hh], false);
        }
        // one word at a time: unpack, then apply it to every head
        const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t v[NP];
          Unpack<BITS>::run(words[w], v);
#pragma unroll
          for (int hh = 0; hh < HPP; ++hh)
#pragma unroll
            for (int k = 0; k < NP; ++k) acc[hh][w * NP + k] = dot2(ps[hh], v[k], acc[hh][w * NP + k]);
        }
      }
      i0 += NBV;
      if (i0 >= n_inst) break;
#pragma unroll
      for (int u = 0; u < NBV; ++u) load(i0 + u, cb[u], mb[u]);
    }
#pragma unroll
    for (int hh = 0; hh < HPP; ++hh) {
      float vals[CPCV];
#pragma unroll
      for (int j = 0; j < CPCV; ++j)
        vals[j] = acc[hh][j] - Unpack<BITS>::offset(j % NP) * sps[hh] + pz[hh];
      wave_reduce_values<D, CPP, CPCV>(W, vals, lane, W.ow + (hp + hh) * (D + 2) + 2);
    }
  }
}

// Values from fp16 rows rows[row0 + i], i < n, probabilities at slots i.
template <int D, int GQ>
__device__ void values_fp16(const DecodeParams& P, const WaveLds& W, const uint16_t* rows,
                            int row0, int n, int lane) {
  constexpr int LT = wave_tokens(GQ) + 4;
  constexpr int CPR = D / 8;
  constexpr int TPI = 64 / CPR;
  const int my_t = lane / CPR, my_c = lane % CPR;
  const int n_inst = (n + TPI - 1) / TPI;
  float acc[GQ][8];
#pragma unroll
  for (int h = 0; h < GQ; ++h)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[h][j] = 0.f;
  auto load = [&](int i) {
    const int t = min(i * TPI + my_t, n - 1);
    return *reinterpret_cast<const uint4*>(rows + int64_t(row0 + t) * D + my_c * 8);
  };
  uint4 buf[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) buf[u] = load(u);
  for (int i0 = 0;;) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int i = i0 + u;
      const uint4 x = buf[u];
      const int t = min(i * TPI + my_t, LT - 1);     // slots past the tokens are zero
      const uint32_t wv[4] = {x.x, x.y, x.z, x.w};
      float f[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[2 * e] = h2f(wv[e] & 0xffffu);
        f[2 * e + 1] = h2f(wv[e] >> 16);
      }
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        const float p = h2f(W.p16[h * LT + t]);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] += p * f[j];
      }
    }
    i0 += NB;
    if (i0 >= n_inst) break;
#pragma unroll
    for (int u = 0; u < NB; ++u) buf[u] = load(i0 + u);
  }
#pragma unroll
  for (int h = 0; h < GQ; ++h) wave_reduce_values<D, CPR, 8>(W, acc[h], lane, W.ow + h * (D + 2) + 2);
}

// ---------------------------------------------------------------------------
// Four waves per SIMD (<= 128 VGPRs) for one query head per kv head: 16
// resident waves per CU keep enough loads in flight to cover HBM latency.
// Grouped heads do GQ times the arithmetic per byte and get 256 VGPRs.
template <int D, int GQ>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(GQ == 1 ? 4 : 2)))
decode_split_kernel(const DecodeParams P) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int LT = wave_tokens(GQ) + 4;
  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform (scalar) so that every loop bound derived from it is scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = blockIdx.x;
  const int64_t stream = blockIdx.y;
  const int b = int(stream / P.Hkv), hkv = int(stream % P.Hkv);

  int ci = 0;
  while (ci + 1 < P.n_cells && P.cells[ci + 1].split0 <= split) ++ci;
  const Cell cell = P.cells[ci];
  const int ST = P.split_tokens;
  const int t0 = cell.t0 + (split - cell.split0) * ST;
  const int t1 = min(t0 + ST, cell.t0 + cell.n);
  const int wt = (ST + kWaves - 1) / kWaves;      // tokens per wave (<= wave_tokens(GQ))
  const int a = min(t0 + wave * wt, t1);
  const int e = min(a + wt, t1);
  const int n = e - a;

  uint16_t* qh16 = reinterpret_cast<uint16_t*>(smem);
  const int64_t qrow = (int64_t(b) * P.Hq + int64_t(hkv) * P.gq) * D;
  for (int i = tid; i < GQ * D; i += NT) {
    const int h = i / D;
    qh16[i] = h < P.gq ? P.q[qrow + i] : uint16_t(0);
  }
  __syncthreads();

  const WaveLds W = carve_wave<D, GQ>(smem, wave);
  // token t of the wave sits at slot slot0 + (t - a); for quantized value runs
  // slot0 makes every value pair block start at an even slot
  int slot0 = 0;
  if (cell.v_src >= 0 && P.v_runs[cell.v_src].bits != 16)
    slot0 = (a - P.v_runs[cell.v_src].tok_begin) & 1;
  if (n > 0) {
    if (cell.k_src >= 0) {
      const Run& run = P.k_runs[cell.k_src];
      const int r0 = a - run.tok_begin, r1 = e - run.tok_begin;
      switch (run.bits) {
        case 2: keys_quantized<D, GQ, 2>(P, W, qh16, stream, run, r0, r1, slot0, lane); break;
        case 4: keys_quantized<D, GQ, 4>(P, W, qh16, stream, run, r0, r1, slot0, lane); break;
        case 8: keys_quantized<D, GQ, 8>(P, W, qh16, stream, run, r0, r1, slot0, lane); break;
        default:
          keys_fp16<D, GQ>(P, W, qh16,
                           reinterpret_cast<const uint16_t*>(P.k_codes + stream * P.k_codes_stride + run.code_off),
                           r0, n, slot0, lane);
      }
    } else {
      keys_fp16<D, GQ>(P, W, qh16, P.k_res + stream * P.k_res_stride, a - P.n_kq, n, slot0, lane);
    }
    wave_lds_sync();

    // softmax state of this wave's range, per head (base-2 logits); every slot
    // of p16 is written, zero outside the wave's tokens
    float mh[GQ], lh[GQ];
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      float mx = -INFINITY;
      for (int i = lane; i < n; i += 64) mx = fmaxf(mx, W.logit[h * LT + slot0 + i]);
      mx = wave_max(mx);
      float sum = 0.f;
      for (int sl = lane; sl < LT; sl += 64) {
        const int i = sl - slot0;
        const float x = (i >= 0 && i < n) ? exp2f(W.logit[h * LT + sl] - mx) : 0.f;
        const uint32_t x16 = f2h(x);
        W.p16[h * LT + sl] = static_cast<uint16_t>(x16);
        sum += h2f(x16);              // the same rounded values the A.V uses
      }
      mh[h] = mx;
      lh[h] = wave_sum(sum);
    }
    wave_lds_sync();

    if (cell.v_src >= 0) {
      const Run& run = P.v_runs[cell.v_src];
      const int r0 = a - run.tok_begin, r1 = e - run.tok_begin;
      switch (run.bits) {
        case 2: values_quantized<D, GQ, 2>(P, W, stream, run, r0, r1, lane); break;
        case 4: values_quantized<D, GQ, 4>(P, W, stream, run, r0, r1, lane); break;
        case 8: values_quantized<D, GQ, 8>(P, W, stream, run, r0, r1, lane); break;
        default:
          values_fp16<D, GQ>(P, W,
                             reinterpret_cast<const uint16_t*>(P.v_codes + stream * P.v_codes_stride + run.code_off),
                             r0, n, lane);
      }
    } else {
      values_fp16<D, GQ>(P, W, P.v_res + stream * P.v_res_stride, a - P.n_vq, n, lane);
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        W.ow[h * (D + 2)] = mh[h];
        W.ow[h * (D + 2) + 1] = lh[h];
      }
    }
  } else {
    for (int i = lane; i < GQ * (D + 2); i += 64) {
      const int j = i % (D + 2);
      W.ow[i] = j == 0 ? -INFINITY : 0.f;
    }
  }
  __syncthreads();

  // combine the waves' states and write this split's partial
  float* ws = P.ws + (stream * P.n_splits + split) * int64_t(P.gq) * (D + 2);
  constexpr DecodeLds lay = decode_lds(D, GQ);
  for (int i = tid; i < P.gq * (D + 2); i += NT) {
    const int h = i / (D + 2), j = i % (D + 2);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float* ow = reinterpret_cast<const float*>(smem + lay.block + w * lay.wave + lay.logit + lay.p16);
      M = fmaxf(M, ow[h * (D + 2)]);
    }
    float r = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float* ow = reinterpret_cast<const float*>(smem + lay.block + w * lay.wave + lay.logit + lay.p16);
      const float f = exp2f(ow[h * (D + 2)] - M);
      r += f * ow[h * (D + 2) + (j == 0 ? 1 : j)];
    }
    ws[i] = j == 0 ? M : r;
  }
}

// Cross-split merge: out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i.
template <int D>
__global__ void __launch_bounds__(D) decode_merge_kernel(const DecodeParams P) {
  const int bh = blockIdx.x;
  const int b = bh / P.Hq, hq = bh % P.Hq;
  const int hkv = hq / P.gq, h = hq % P.gq;
  const int64_t stream = int64_t(b) * P.Hkv + hkv;
  const int64_t step = int64_t(P.gq) * (D + 2);
  const float* w = P.ws + stream * P.n_splits * step + int64_t(h) * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < P.n_splits; ++s) M = fmaxf(M, w[s * step]);
  float den = 0.f, num = 0.f;
  const int c = threadIdx.x;
  for (int s = 0; s < P.n_splits; ++s) {
    const float f = exp2f(w[s * step] - M);
    den += f * w[s * step + 1];
    num += f * w[s * step + 2 + c];
  }
  P.out[(int64_t(b) * P.Hq + hq) * D + c] = num / den;
}

template <int D, int GQ>
hipError_t launch_dg(const DecodeParams& p, hipStream_t s) {
  const size_t lds = size_t(decode_lds(D, GQ).total);
  hipLaunchKernelGGL((decode_split_kernel<D, GQ>), dim3(p.n_splits, p.B * p.Hkv), dim3(NT),
                     lds, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(p.B * p.Hq), dim3(D), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeParams& p, int GQ, hipStream_t s) {
  switch (GQ) {
    case 1: return launch_dg<D, 1>(p, s);
    case 2: return launch_dg<D, 2>(p, s);
    case 4: return launch_dg<D, 4>(p, s);
    case 8: return launch_dg<D, 8>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int GQ, hipStream_t s) {
  switch (p.D) {
    case 64: return launch_d<64>(p, GQ, s);
    case 128: return launch_d<128>(p, GQ, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
