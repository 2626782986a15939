// Group quantize + pack + append kernels, and the fp16 row copy.
//
// Quantizer: asymmetric round-to-nearest, Q = round((x - z)/s), x' = Q*s + z
// (KIVI note, "How it works"; WindowQuant Sec. 3.3.3, Eq. 14-16), with
// s = (max - min)/(2^b - 1) and z = min stored as fp16 and the stored values
// used to encode.  Keys: one group per channel over G consecutive tokens;
// values: one group per token over G consecutive channels (KIVI note,
// "Method details" and Algorithm 1).
//
// Bit-exact contract (include/kvq.h): every step is one IEEE fp32 operation
// on fp16-exact inputs -- subtract, correctly rounded divide, round half to
// even -- so this file is built without FMA contraction and with correctly
// rounded fp32 division.  The wave kernels and the decode-step append take
// the codes from a reciprocal product and divide only where that could
// change a code (encode_fast, kvq_quant.h).

#include "kvq_internal.h"
#include "kvq_device.h"
#include "kvq_quant.h"

namespace kvq {
namespace {

// Keys, one thread per channel (block = one group of G tokens of one
// stream): the shape whose rows do not fit in one wave's registers (d_h 128
// with groups of 128 tokens).
template <int BITS>
__global__ void __launch_bounds__(128) quantize_keys_kernel(QuantParams p) {
  __shared__ uint8_t codes[128 * 128];  // [token in group][channel]
  const int c = threadIdx.x;
  const int j = blockIdx.x;
  const int64_t s = blockIdx.y;
  const int G = p.G, D = p.D;
  const uint16_t* src = p.src + s * p.src_stream_stride;
  float mn = INFINITY, mx = -INFINITY;
  for (int i = 0; i < G; ++i) {
    const int tok = j * G + i;
    const int64_t row = p.src_rows ? p.src_rows[tok] : tok;
    const float x = h2f(src[row * p.src_row_stride + c]);
    mn = fminf(mn, x);
    mx = fmaxf(mx, x);
  }
  const GroupScale g = group_scale<BITS>(mn, mx);
  uint32_t* meta = reinterpret_cast<uint32_t*>(p.meta + s * p.meta_stream_stride);
  meta[int64_t(p.dst_tok / G + j) * D + c] = g.s16 | (g.z16 << 16);
  for (int i = 0; i < G; ++i) {
    const int tok = j * G + i;
    const int64_t row = p.src_rows ? p.src_rows[tok] : tok;
    codes[i * D + c] = static_cast<uint8_t>(encode<BITS>(h2f(src[row * p.src_row_stride + c]), g));
  }
  __syncthreads();
  constexpr int kCpw = 32 / BITS;       // channels per 32-bit word
  const int wpr = D / kCpw;             // words per row
  const int64_t rb = int64_t(D) * BITS / 8;
  uint8_t* out = p.codes + s * p.codes_stream_stride;
  for (int wi = c; wi < G * wpr; wi += blockDim.x) {
    const int i = wi / wpr, wr = wi % wpr;
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < kCpw; ++k)
      word |= uint32_t(codes[i * D + wr * kCpw + k]) << (k * BITS);
    *reinterpret_cast<uint32_t*>(out + int64_t(p.dst_tok + j * G + i) * rb + wr * 4) = word;
  }
}

// ---------------------------------------------------------------------------
// Wave-cooperative quantizers (HBM-bound shapes).  A lane holds 8 channels
// (16 bytes) of a row; D/8 lanes cover a row.  Source rows are read once with
// the non-temporal cache policy; codes are assembled in registers so that
// each store instruction covers whole rows (keys) or whole token-pair blocks
// (values).

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

typedef const __attribute__((address_space(1))) u32x4* global_u32x4_ptr;

// 16 bytes of a source row (device memory: a global, not a flat, load)
__device__ __forceinline__ uint4 load_row16(const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load((global_u32x4_ptr)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// min / max over the lanes l, l ^ LPR, l ^ 2 LPR, ... (the rows of a load
// instruction that hold the same 8 channels) of packed fp16 pairs; every
// lane gets the result.
template <int LPR>
__device__ __forceinline__ uint32_t rows_min(uint32_t x) {
  if constexpr (LPR == 8) x = pk_min_f16(x, __builtin_amdgcn_update_dpp(x, x, 0x128, 0xF, 0xF, false));  // row_ror:8
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = pk_min_f16(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return pk_min_f16(b[0], b[1]);
}
template <int LPR>
__device__ __forceinline__ uint32_t rows_max(uint32_t x) {
  if constexpr (LPR == 8) x = pk_max_f16(x, __builtin_amdgcn_update_dpp(x, x, 0x128, 0xF, 0xF, false));
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = pk_max_f16(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return pk_max_f16(b[0], b[1]);
}

// min / max over aligned groups of N consecutive lanes (N = 2 .. 16) of
// packed fp16 pairs: DPP quad permutations, then half-row and row mirrors.
template <int N>
__device__ __forceinline__ uint32_t group_pk_min(uint32_t x) {
  if (N >= 2) x = pk_min_f16(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false));
  if (N >= 4) x = pk_min_f16(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false));
  if (N >= 8) x = pk_min_f16(x, __builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false));
  if (N >= 16) x = pk_min_f16(x, __builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false));
  return x;
}
template <int N>
__device__ __forceinline__ uint32_t group_pk_max(uint32_t x) {
  if (N >= 2) x = pk_max_f16(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false));
  if (N >= 4) x = pk_max_f16(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false));
  if (N >= 8) x = pk_max_f16(x, __builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false));
  if (N >= 16) x = pk_max_f16(x, __builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false));
  return x;
}

// (low half of a, low half of b) and (high half of a, high half of b)
__device__ __forceinline__ uint32_t lows(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t highs(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

__device__ __forceinline__ uint32_t word(const uint4& x, int e) {
  return e == 0 ? x.x : e == 1 ? x.y : e == 2 ? x.z : x.w;
}

// Keys: one wave per (stream, key group of G tokens).  Load instruction k
// brings rows k*RPI .. k*RPI + RPI-1 of the group, lane l holding channels
// 8*(l % LPR) .. +7 of row k*RPI + l / LPR.  Channel extrema: over the lane's
// NL rows on packed fp16 pairs, then across the RPI lanes of the same
// channels.  Every lane encodes its 8 channels of its NL rows into 8*BITS
// bits per row (codes8_fast; a row batch of the wave that it cannot decide,
// or a wave with a group scale outside scale_unclamped, by codes8_exact).
template <int BITS, int D, int G>
__global__ void __launch_bounds__(256) quantize_keys_wave_kernel(QuantParams p) {
  constexpr int LPR = D / 8;
  constexpr int RPI = 64 / LPR;
  constexpr int NL = G / RPI;
  constexpr int64_t RB = int64_t(D) * BITS / 8;
  const int lane = threadIdx.x & 63;
  const int j = int(blockIdx.x) * 4 + int(threadIdx.x >> 6);   // key group of the stream
  if (j >= p.n_tok / G) return;                                 // uniform per wave
  const int64_t s = blockIdx.y;
  const int c8 = lane % LPR, r0 = lane / LPR;
  const uint16_t* src = p.src + s * p.src_stream_stride + c8 * 8;
  // row indices first (one uniform branch), then the NL loads back to back:
  // a gather read inside the load loop would split it into blocks that each
  // wait for the previous load
  const uint16_t* rp[NL];
  if (p.src_rows) {
#pragma unroll
    for (int k = 0; k < NL; ++k) rp[k] = src + int64_t(p.src_rows[j * G + k * RPI + r0]) * p.src_row_stride;
  } else {
    const int64_t step = int64_t(RPI) * p.src_row_stride;
    rp[0] = src + int64_t(j * G + r0) * p.src_row_stride;
#pragma unroll
    for (int k = 1; k < NL; ++k) rp[k] = rp[k - 1] + step;
  }
  uint4 x[NL];
#pragma unroll
  for (int k = 0; k < NL; ++k) x[k] = load_row16(rp[k]);
  uint32_t mnw[4], mxw[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) mnw[e] = mxw[e] = word(x[0], e);
#pragma unroll
  for (int k = 1; k < NL; ++k) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mnw[e] = pk_min_f16(mnw[e], word(x[k], e));
      mxw[e] = pk_max_f16(mxw[e], word(x[k], e));
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    mnw[e] = rows_min<LPR>(mnw[e]);
    mxw[e] = rows_max<LPR>(mxw[e]);
  }
  GroupScale gs[8];
  float z[8], inv[8];
  bool slow = false;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    gs[2 * e] = group_scale<BITS>(h2f(mnw[e] & 0xffffu), h2f(mxw[e] & 0xffffu));
    gs[2 * e + 1] = group_scale<BITS>(h2f(mnw[e] >> 16), h2f(mxw[e] >> 16));
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    z[c] = gs[c].z;
    inv[c] = gs[c].inv;
    slow |= !scale_unclamped(gs[c].s16);
  }
  const float one = 1.0f;
  // row k's 8 channels (BITS bytes) at a constant offset from the lane's first row
  uint8_t* out = p.codes + s * p.codes_stream_stride + c8 * BITS + int64_t(p.dst_tok + j * G + r0) * RB;
#pragma unroll
  for (int k = 0; k < NL; ++k) {
    uint32_t ch[BITS / 2];
    float err = 0.0f;
    codes8_fast<BITS>(x[k], z, inv, one, err, ch);
    if (wave_any(slow || err >= kFastFar<BITS>)) codes8_exact<BITS>(x[k], gs, ch);   // uniform, rare
    uint8_t* dst = out + k * RPI * RB;
    if constexpr (BITS == 2) *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>(ch[0]);
    else if constexpr (BITS == 4) *reinterpret_cast<uint32_t*>(dst) = ch[0] | (ch[1] << 16);
    else *reinterpret_cast<uint2*>(dst) = make_uint2(ch[0] | (ch[1] << 16), ch[2] | (ch[3] << 16));
  }
  if (r0 == 0) {
    uint4* meta = reinterpret_cast<uint4*>(p.meta + s * p.meta_stream_stride +
                                           (int64_t(p.dst_tok / G + j) * D + c8 * 8) * 4);
    meta[0] = make_uint4(gs[0].s16 | (gs[0].z16 << 16), gs[1].s16 | (gs[1].z16 << 16),
                         gs[2].s16 | (gs[2].z16 << 16), gs[3].s16 | (gs[3].z16 << 16));
    meta[1] = make_uint4(gs[4].s16 | (gs[4].z16 << 16), gs[5].s16 | (gs[5].z16 << 16),
                         gs[6].s16 | (gs[6].z16 << 16), gs[7].s16 | (gs[7].z16 << 16));
  }
}

// Values: one wave per PPW = 4 * (64 / LPR) token-pair blocks of a stream.
// Lane l handles channels 8*(l % LPR) .. +7 of both tokens of one pair block:
// its 16-bit units of token 2P (low halves) and 2P+1 (high halves) form BITS/2
// whole words of the block.  Group extrema per token come from the G/8
// consecutive lanes of the group.  A block whose low token precedes this call
// (dst_tok odd) gets only its high halves; a block whose high token follows
// the last appended one gets a zero high half and a zero (scale, zero) pair.
template <int BITS, int D, int G>
__global__ void __launch_bounds__(256) quantize_values_pairs_kernel(QuantParams p) {
  constexpr int LPR = D / 8;
  constexpr int PPI = 64 / LPR;         // pair blocks per instruction
  constexpr int U = 4;                  // instructions per wave
  constexpr int PPW = PPI * U;
  constexpr int NG = D / G;
  constexpr int LPG = G / 8;            // lanes per group
  constexpr int64_t RB = int64_t(D) * BITS / 8;
  constexpr int WPL = BITS / 2;         // words of a pair block per lane
  constexpr int KPU = 16 / BITS;        // codes per 16-bit unit
  const int lane = threadIdx.x & 63;
  const int64_t s = blockIdx.y;
  const int64_t p_lo = p.dst_tok >> 1;
  const int64_t p_hi = (int64_t(p.dst_tok) + p.n_tok - 1) >> 1;
  const int64_t P0 = p_lo + (int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6)) * PPW;
  if (P0 > p_hi) return;                // uniform per wave
  const int c8 = lane % LPR, pl = lane / LPR;
  const uint16_t* src = p.src + s * p.src_stream_stride + c8 * 8;
  // source rows of the pair blocks' tokens (an absent token reads source
  // row 0, which always exists, and is zeroed after the load), resolved
  // before the loads so that all 2U of them issue back to back
  int64_t ia[U], ib[U];
  bool ha[U], hb[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t P = P0 + u * PPI + pl;
    const int64_t i0 = 2 * P - p.dst_tok, i1 = i0 + 1;
    ha[u] = P <= p_hi && i0 >= 0;
    hb[u] = P <= p_hi && i1 < p.n_tok;
    ia[u] = ha[u] ? i0 : 0;
    ib[u] = hb[u] ? i1 : 0;
  }
  if (p.src_rows) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      ia[u] = p.src_rows[ia[u]];
      ib[u] = p.src_rows[ib[u]];
    }
  }
  uint4 xa[U], xb[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    xa[u] = load_row16(src + ia[u] * p.src_row_stride);
    xb[u] = load_row16(src + ib[u] * p.src_row_stride);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!ha[u]) xa[u] = make_uint4(0, 0, 0, 0);
    if (!hb[u]) xb[u] = make_uint4(0, 0, 0, 0);
  }
  uint8_t* codes = p.codes + s * p.codes_stream_stride;
  uint8_t* meta = p.meta + s * p.meta_stream_stride;
  const int g = c8 / LPG;
  const float one = 1.0f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t P = P0 + u * PPI + pl;
    const int64_t i0 = 2 * P - p.dst_tok, i1 = i0 + 1;
    const bool va = i0 >= 0, vb = i1 < p.n_tok;   // meaningful only for P <= p_hi
    // token extrema on packed fp16 pairs: over the lane's 8 channels (its 4
    // words, then the two halves, tokens a and b side by side in one word),
    // then over the LPG lanes of the group
    const uint32_t ma = pk_min_f16(pk_min_f16(xa[u].x, xa[u].y), pk_min_f16(xa[u].z, xa[u].w));
    const uint32_t Ma = pk_max_f16(pk_max_f16(xa[u].x, xa[u].y), pk_max_f16(xa[u].z, xa[u].w));
    const uint32_t mb = pk_min_f16(pk_min_f16(xb[u].x, xb[u].y), pk_min_f16(xb[u].z, xb[u].w));
    const uint32_t Mb = pk_max_f16(pk_max_f16(xb[u].x, xb[u].y), pk_max_f16(xb[u].z, xb[u].w));
    const uint32_t mn2 = group_pk_min<LPG>(pk_min_f16(lows(ma, mb), highs(ma, mb)));
    const uint32_t mx2 = group_pk_max<LPG>(pk_max_f16(lows(Ma, Mb), highs(Ma, Mb)));
    GroupScale ga[8], gb[8];
    ga[0] = group_scale<BITS>(h2f(mn2 & 0xffffu), h2f(mx2 & 0xffffu));
    gb[0] = group_scale<BITS>(h2f(mn2 >> 16), h2f(mx2 >> 16));
    float za[8], inva[8], zb[8], invb[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      ga[c] = ga[0];
      gb[c] = gb[0];
      za[c] = ga[0].z;
      inva[c] = ga[0].inv;
      zb[c] = gb[0].z;
      invb[c] = gb[0].inv;
    }
    uint32_t cha[WPL], chb[WPL];
    float err = 0.0f;
    codes8_fast<BITS>(xa[u], za, inva, one, err, cha);
    codes8_fast<BITS>(xb[u], zb, invb, one, err, chb);
    const bool slow = !scale_unclamped(ga[0].s16) || !scale_unclamped(gb[0].s16);
    if (wave_any(slow || err >= kFastFar<BITS>)) {   // uniform, rare
      codes8_exact<BITS>(xa[u], ga, cha);
      codes8_exact<BITS>(xb[u], gb, chb);
    }
    uint32_t w[WPL];
#pragma unroll
    for (int k = 0; k < WPL; ++k) w[k] = cha[k] | (vb ? chb[k] << 16 : 0u);
    if (P > p_hi) continue;
    uint8_t* blk = codes + P * 2 * RB + c8 * WPL * 4;
    const bool lead = (c8 % LPG) == 0;
    uint32_t* mp = reinterpret_cast<uint32_t*>(meta + (P * NG + g) * 8);
    if (va) {
      if constexpr (WPL == 1) *reinterpret_cast<uint32_t*>(blk) = w[0];
      else if constexpr (WPL == 2) *reinterpret_cast<uint2*>(blk) = make_uint2(w[0], w[1]);
      else *reinterpret_cast<uint4*>(blk) = make_uint4(w[0], w[1], w[2], w[3]);
      if (lead)
        *reinterpret_cast<uint2*>(mp) =
            make_uint2(ga[0].s16 | (ga[0].z16 << 16), vb ? (gb[0].s16 | (gb[0].z16 << 16)) : 0u);
    } else {
#pragma unroll
      for (int k = 0; k < WPL; ++k) reinterpret_cast<uint16_t*>(blk)[2 * k + 1] = static_cast<uint16_t>(w[k] >> 16);
      if (lead) mp[1] = gb[0].s16 | (gb[0].z16 << 16);
    }
  }
}

// One decode step's append (KIVI note, Algorithm 1, Decoding), one launch,
// one wave per stream: the new key and value rows are copied (16 bytes per
// lane), and (v_quant_row >= 0) one value-window row is quantized with each
// lane holding D/64 channels: group min/max by cross-lane reductions, codes
// from the same group_scale/encode as quantize_values_pairs_kernel, 16-bit units
// assembled by OR across the lanes of a unit.
template <int BITS, int D, int G>
__global__ void __launch_bounds__(256) decode_append_kernel(AppendParams p) {
  const int64_t s = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (s >= p.n_streams) return;          // uniform per wave
  append_stream<BITS, D, G>(p, s, int(threadIdx.x & 63));
}

// fp16 row copy, 16 bytes per thread.
__global__ void __launch_bounds__(256) copy_rows_kernel(
    const uint16_t* src, int64_t sss, int64_t srs, const int32_t* rows, uint8_t* dst,
    int64_t dss, int32_t row0, int32_t n_streams, int32_t D, int32_t n_rows) {
  const int cpr = D / 8;
  const int64_t item = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = int64_t(n_streams) * n_rows * cpr;
  if (item >= total) return;
  const int c = int(item % cpr);
  const int64_t rest = item / cpr;
  const int i = int(rest % n_rows);
  const int64_t s = rest / n_rows;
  const int64_t r = rows ? rows[i] : i;
  const uint4 v = *reinterpret_cast<const uint4*>(src + s * sss + r * srs + c * 8);
  *reinterpret_cast<uint4*>(dst + s * dss + int64_t(row0 + i) * D * 2 + c * 16) = v;
}

}  // namespace

template <int BITS, int D, int G>
hipError_t launch_keys_bdg(const QuantParams& p, hipStream_t s) {
  const int n_groups = p.n_tok / G;
  hipLaunchKernelGGL((quantize_keys_wave_kernel<BITS, D, G>), dim3(unsigned((n_groups + 3) / 4), p.n_streams),
                     dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int BITS, int D>
hipError_t launch_keys_bd(const QuantParams& p, hipStream_t s) {
  switch (p.G) {
    case 32: return launch_keys_bdg<BITS, D, 32>(p, s);
    case 64: return launch_keys_bdg<BITS, D, 64>(p, s);
    case 128:
      if constexpr (D == 64) return launch_keys_bdg<BITS, D, 128>(p, s);
      // 32 rows per lane would not fit in registers: one thread per channel
      hipLaunchKernelGGL(quantize_keys_kernel<BITS>, dim3(p.n_tok / p.G, p.n_streams), dim3(p.D), 0, s, p);
      return hipGetLastError();
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_quantize_keys(const QuantParams& p, hipStream_t s) {
  switch (p.bits * 1000 + p.D) {
    case 2064: return launch_keys_bd<2, 64>(p, s);
    case 2128: return launch_keys_bd<2, 128>(p, s);
    case 4064: return launch_keys_bd<4, 64>(p, s);
    case 4128: return launch_keys_bd<4, 128>(p, s);
    case 8064: return launch_keys_bd<8, 64>(p, s);
    case 8128: return launch_keys_bd<8, 128>(p, s);
    default: return hipErrorInvalidValue;
  }
}

template <int BITS, int D, int G>
hipError_t launch_values_bdg(const QuantParams& p, hipStream_t s) {
  constexpr int PPW = 4 * (64 / (D / 8));
  const int64_t pairs = ((int64_t(p.dst_tok) + p.n_tok - 1) >> 1) - (p.dst_tok >> 1) + 1;
  const int64_t waves = (pairs + PPW - 1) / PPW;
  hipLaunchKernelGGL((quantize_values_pairs_kernel<BITS, D, G>), dim3(unsigned((waves + 3) / 4), p.n_streams),
                     dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int BITS, int D>
hipError_t launch_values_bd(const QuantParams& p, hipStream_t s) {
  switch (p.G) {
    case 32: return launch_values_bdg<BITS, D, 32>(p, s);
    case 64: return launch_values_bdg<BITS, D, 64>(p, s);
    case 128:
      if constexpr (D == 128) return launch_values_bdg<BITS, D, 128>(p, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_quantize_values(const QuantParams& p, hipStream_t s) {
  switch (p.bits * 1000 + p.D) {
    case 2064: return launch_values_bd<2, 64>(p, s);
    case 2128: return launch_values_bd<2, 128>(p, s);
    case 4064: return launch_values_bd<4, 64>(p, s);
    case 4128: return launch_values_bd<4, 128>(p, s);
    case 8064: return launch_values_bd<8, 64>(p, s);
    case 8128: return launch_values_bd<8, 128>(p, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int G>
hipError_t launch_append_dg(const AppendParams& p, hipStream_t s) {
  const dim3 grid(unsigned((p.n_streams + 3) / 4)), block(256);
  switch (p.bits) {
    case 2: hipLaunchKernelGGL((decode_append_kernel<2, D, G>), grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL((decode_append_kernel<4, D, G>), grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL((decode_append_kernel<8, D, G>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_append(const AppendParams& p, hipStream_t s) {
  switch (p.D * 1000 + p.G) {
    case 64032: return launch_append_dg<64, 32>(p, s);
    case 64064: return launch_append_dg<64, 64>(p, s);
    case 128032: return launch_append_dg<128, 32>(p, s);
    case 128064: return launch_append_dg<128, 64>(p, s);
    case 128128: return launch_append_dg<128, 128>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_copy_rows(const uint16_t* src, int64_t src_stream_stride,
                            int64_t src_row_stride, const int32_t* rows,
                            uint8_t* dst, int64_t dst_stream_bytes, int32_t dst_row0,
                            int32_t n_streams, int32_t D, int32_t n_rows, hipStream_t s) {
  const int64_t total = int64_t(n_streams) * n_rows * (D / 8);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_rows_kernel, dim3(unsigned((total + 255) / 256)), dim3(256), 0, s,
                     src, src_stream_stride, src_row_stride, rows, dst, dst_stream_bytes,
                     dst_row0, n_streams, D, n_rows);
  return hipGetLastError();
}

}  // namespace kvq
