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
// rounded fp32 division.

#include "kvq_internal.h"
#include "kvq_device.h"
#include "kvq_quant.h"

namespace kvq {
namespace {

// Keys: block = one group of G tokens of one stream, thread = channel.
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

// Values: one group (G channels at x) of the token with index te of a value
// run.  The codes go to the token's 16-bit halves of its pair block in
// `codes` (the run's arena of this stream), the (scale, zero) pair to `meta`.
// `last`: the token is the last one appended; at an even index its pair
// partner is not written yet, so the partner's halves and (scale, zero) are
// zeroed and decode reads finite values (the next append overwrites them).
template <int BITS>
__device__ __forceinline__ void quantize_value_group(const uint16_t* x, int G, int g, int NG, int D,
                                                     int64_t te, bool last, uint8_t* codes,
                                                     uint32_t* meta) {
  // the group's G fp16 values stay in registers (G <= 128: 16 loads of 16 B)
  uint32_t xw[64];
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    if (k * 8 >= G) break;
    const uint4 u = *reinterpret_cast<const uint4*>(x + k * 8);
    xw[4 * k] = u.x; xw[4 * k + 1] = u.y; xw[4 * k + 2] = u.z; xw[4 * k + 3] = u.w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = h2f(xw[4 * k + e] & 0xffffu), b = h2f(xw[4 * k + e] >> 16);
      mn = fminf(mn, fminf(a, b));
      mx = fmaxf(mx, fmaxf(a, b));
    }
  }
  const GroupScale gs = group_scale<BITS>(mn, mx);
  const int64_t pair = te >> 1;
  const int par = int(te & 1);
  const int64_t rb = int64_t(D) * BITS / 8;
  uint8_t* blk = codes + pair * 2 * rb;
  constexpr int kPerUnit = 16 / BITS;   // codes per 16-bit unit
  const int units = G / kPerUnit;
  const int u0 = g * units;
#pragma unroll
  for (int u = 0; u < 128 / kPerUnit; ++u) {
    if (u >= units) break;
    uint32_t unit = 0;
#pragma unroll
    for (int k = 0; k < kPerUnit; ++k) {
      const int e = u * kPerUnit + k;                 // element of the group
      const uint32_t h = (xw[e >> 1] >> (16 * (e & 1))) & 0xffffu;
      unit |= encode<BITS>(h2f(h), gs) << (k * BITS);
    }
    *reinterpret_cast<uint16_t*>(blk + 4 * (u0 + u) + 2 * par) = static_cast<uint16_t>(unit);
  }
  meta[(pair * NG + g) * 2 + par] = gs.s16 | (gs.z16 << 16);
  if (par == 0 && last) {
    for (int u = 0; u < units; ++u)
      *reinterpret_cast<uint16_t*>(blk + 4 * (u0 + u) + 2) = 0;
    meta[(pair * NG + g) * 2 + 1] = 0u;
  }
}

// Values: thread = one group (G channels) of one token of one stream.
template <int BITS>
__global__ void __launch_bounds__(256) quantize_values_kernel(QuantParams p, int NG) {
  const int64_t item = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = int64_t(p.n_streams) * p.n_tok * NG;
  if (item >= total) return;
  const int g = int(item % NG);
  const int64_t rest = item / NG;
  const int i = int(rest % p.n_tok);
  const int64_t s = rest / p.n_tok;
  const int64_t row = p.src_rows ? p.src_rows[i] : i;
  const uint16_t* x = p.src + s * p.src_stream_stride + row * p.src_row_stride + int64_t(g) * p.G;
  quantize_value_group<BITS>(x, p.G, g, NG, p.D, int64_t(p.dst_tok) + i, i == p.n_tok - 1,
                             p.codes + s * p.codes_stream_stride,
                             reinterpret_cast<uint32_t*>(p.meta + s * p.meta_stream_stride));
}

// One decode step's append (KIVI note, Algorithm 1, Decoding), one launch,
// one wave per stream: the new key and value rows are copied (16 bytes per
// lane), and (v_quant_row >= 0) one value-window row is quantized with each
// lane holding D/64 channels: group min/max by cross-lane reductions, codes
// from the same group_scale/encode as quantize_value_group, 16-bit units
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

hipError_t launch_quantize_keys(const QuantParams& p, hipStream_t s) {
  const dim3 grid(p.n_tok / p.G, p.n_streams), block(p.D);
  switch (p.bits) {
    case 2: hipLaunchKernelGGL(quantize_keys_kernel<2>, grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL(quantize_keys_kernel<4>, grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL(quantize_keys_kernel<8>, grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_quantize_values(const QuantParams& p, hipStream_t s) {
  const int NG = p.D / p.G;
  const int64_t total = int64_t(p.n_streams) * p.n_tok * NG;
  const dim3 grid(unsigned((total + 255) / 256)), block(256);
  switch (p.bits) {
    case 2: hipLaunchKernelGGL(quantize_values_kernel<2>, grid, block, 0, s, p, NG); break;
    case 4: hipLaunchKernelGGL(quantize_values_kernel<4>, grid, block, 0, s, p, NG); break;
    case 8: hipLaunchKernelGGL(quantize_values_kernel<8>, grid, block, 0, s, p, NG); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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
