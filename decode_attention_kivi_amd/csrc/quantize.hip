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

__device__ __forceinline__ uint4 load_row16(const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void halves(const uint4& x, float (&f)[8]) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = h2f(w[e] & 0xffffu);
    f[2 * e + 1] = h2f(w[e] >> 16);
  }
}

// min / max over the lanes l, l ^ LPR, l ^ 2 LPR, ... (the rows of a load
// instruction that hold the same 8 channels), every lane gets the result.
template <int LPR>
__device__ __forceinline__ float rows_min(float x) {
  if constexpr (LPR == 8) x = fminf(x, __builtin_amdgcn_update_dpp(x, x, 0x128, 0xF, 0xF, false));  // row_ror:8
  const auto a = __builtin_amdgcn_permlane16_swap(fbits(x), fbits(x), false, false);
  x = fminf(bitsf(a[0]), bitsf(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(fbits(x), fbits(x), false, false);
  return fminf(bitsf(b[0]), bitsf(b[1]));
}
template <int LPR>
__device__ __forceinline__ float rows_max(float x) {
  if constexpr (LPR == 8) x = fmaxf(x, __builtin_amdgcn_update_dpp(x, x, 0x128, 0xF, 0xF, false));
  const auto a = __builtin_amdgcn_permlane16_swap(fbits(x), fbits(x), false, false);
  x = fmaxf(bitsf(a[0]), bitsf(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(fbits(x), fbits(x), false, false);
  return fmaxf(bitsf(b[0]), bitsf(b[1]));
}

// Keys: one wave per (stream, key group of G tokens).  Load instruction k
// brings rows k*RPI .. k*RPI + RPI-1 of the group, lane l holding channels
// 8*(l % LPR) .. +7 of row k*RPI + l / LPR.  Channel extrema: over the lane's
// NL rows, then across the RPI lanes of the same channels.  Every lane
// encodes its 8 channels of its NL rows into 8*BITS bits per row.
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
  uint4 x[NL];
#pragma unroll
  for (int k = 0; k < NL; ++k) {
    const int tok = j * G + k * RPI + r0;
    const int64_t row = p.src_rows ? p.src_rows[tok] : tok;
    x[k] = load_row16(src + row * p.src_row_stride);
  }
  float mn[8], mx[8];
  {
    float f[8];
    halves(x[0], f);
#pragma unroll
    for (int c = 0; c < 8; ++c) mn[c] = mx[c] = f[c];
  }
#pragma unroll
  for (int k = 1; k < NL; ++k) {
    float f[8];
    halves(x[k], f);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      mn[c] = fminf(mn[c], f[c]);
      mx[c] = fmaxf(mx[c], f[c]);
    }
  }
  GroupScale gs[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) gs[c] = group_scale<BITS>(rows_min<LPR>(mn[c]), rows_max<LPR>(mx[c]));
  uint8_t* out = p.codes + s * p.codes_stream_stride + c8 * BITS;   // 8 channels = BITS bytes
#pragma unroll
  for (int k = 0; k < NL; ++k) {
    float f[8];
    halves(x[k], f);
    uint32_t lo = 0, hi = 0;
    bool near = false;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t q = encode_fast<BITS>(f[c], gs[c], near);
      const int bit = c * BITS;
      if (bit < 32) lo |= q << bit;
      else hi |= q << (bit - 32);
    }
    if (wave_any(near)) {                // (uniform, rare) a quotient near a rounding boundary
      lo = hi = 0;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t q = encode<BITS>(f[c], gs[c]);
        const int bit = c * BITS;
        if (bit < 32) lo |= q << bit;
        else hi |= q << (bit - 32);
      }
    }
    uint8_t* dst = out + int64_t(p.dst_tok + j * G + k * RPI + r0) * RB;
    if constexpr (BITS == 2) *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>(lo);
    else if constexpr (BITS == 4) *reinterpret_cast<uint32_t*>(dst) = lo;
    else *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
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
  uint4 xa[U], xb[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t P = P0 + u * PPI + pl;
    const int64_t i0 = 2 * P - p.dst_tok, i1 = i0 + 1;
    xa[u] = make_uint4(0, 0, 0, 0);
    xb[u] = make_uint4(0, 0, 0, 0);
    if (P <= p_hi && i0 >= 0) {
      const int64_t row = p.src_rows ? p.src_rows[i0] : i0;
      xa[u] = load_row16(src + row * p.src_row_stride);
    }
    if (P <= p_hi && i1 < p.n_tok) {
      const int64_t row = p.src_rows ? p.src_rows[i1] : i1;
      xb[u] = load_row16(src + row * p.src_row_stride);
    }
  }
  uint8_t* codes = p.codes + s * p.codes_stream_stride;
  uint8_t* meta = p.meta + s * p.meta_stream_stride;
  const int g = c8 / LPG;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t P = P0 + u * PPI + pl;
    const int64_t i0 = 2 * P - p.dst_tok, i1 = i0 + 1;
    const bool va = i0 >= 0, vb = i1 < p.n_tok;   // meaningful only for P <= p_hi
    float fa[8], fb[8];
    halves(xa[u], fa);
    halves(xb[u], fb);
    float mna = fa[0], mxa = fa[0], mnb = fb[0], mxb = fb[0];
#pragma unroll
    for (int c = 1; c < 8; ++c) {
      mna = fminf(mna, fa[c]); mxa = fmaxf(mxa, fa[c]);
      mnb = fminf(mnb, fb[c]); mxb = fmaxf(mxb, fb[c]);
    }
    const GroupScale ga = group_scale<BITS>(group_min<LPG>(mna), group_max<LPG>(mxa));
    const GroupScale gb = group_scale<BITS>(group_min<LPG>(mnb), group_max<LPG>(mxb));
    uint32_t w[WPL];
#pragma unroll
    for (int k = 0; k < WPL; ++k) w[k] = 0;
    bool near = false;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int k = c / KPU, sh = (c % KPU) * BITS;
      w[k] |= encode_fast<BITS>(fa[c], ga, near) << sh;
      if (vb) w[k] |= encode_fast<BITS>(fb[c], gb, near) << (16 + sh);
    }
    if (wave_any(near)) {                // (uniform, rare) a quotient near a rounding boundary
#pragma unroll
      for (int k = 0; k < WPL; ++k) w[k] = 0;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int k = c / KPU, sh = (c % KPU) * BITS;
        w[k] |= encode<BITS>(fa[c], ga) << sh;
        if (vb) w[k] |= encode<BITS>(fb[c], gb) << (16 + sh);
      }
    }
    if (P > p_hi) continue;
    uint8_t* blk = codes + P * 2 * RB + c8 * WPL * 4;
    const bool lead = (c8 % LPG) == 0;
    uint32_t* mp = reinterpret_cast<uint32_t*>(meta + (P * NG + g) * 8);
    if (va) {
      if constexpr (WPL == 1) *reinterpret_cast<uint32_t*>(blk) = w[0];
      else if constexpr (WPL == 2) *reinterpret_cast<uint2*>(blk) = make_uint2(w[0], w[1]);
      else *reinterpret_cast<uint4*>(blk) = make_uint4(w[0], w[1], w[2], w[3]);
      if (lead)
        *reinterpret_cast<uint2*>(mp) = make_uint2(ga.s16 | (ga.z16 << 16), vb ? (gb.s16 | (gb.z16 << 16)) : 0u);
    } else {
#pragma unroll
      for (int k = 0; k < WPL; ++k) reinterpret_cast<uint16_t*>(blk)[2 * k + 1] = static_cast<uint16_t>(w[k] >> 16);
      if (lead) mp[1] = gb.s16 | (gb.z16 << 16);
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
