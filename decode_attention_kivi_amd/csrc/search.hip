// WindowQuant window-level quantization search (ACM TACO, Sec. 3.2): each
// visual window's score is the mean cosine similarity between the prompt's
// text tokens and the window's visual tokens (Eq. 8); the score picks fp16,
// int4 or int2 against the layer's two thresholds (Sec. 3.2.1, Eq. 10-11),
// the first window stays fp16 (Sec. 3.2.2), and a batch shares one
// configuration, each window taking the width most of its requests chose
// (Sec. 3.2.3).
//
// The mean over all N*S pairs of unit vectors is the dot product of the two
// sums of unit vectors divided by N*S, so the whole search is one streaming
// pass over the tokens:
//   search_sums_kernel   one workgroup per (chunk of <= kChunk tokens of one
//                        window or of the prompt, batch row): every token
//                        row is normalized by one wave (a DPP sum of squares)
//                        and added into the wave's fp32 sum; the four waves'
//                        sums are added in LDS in wave order and the chunk
//                        sum goes to the workspace;
//   search_vote_kernel   one workgroup per window: the chunk sums of the
//                        window and of the prompt, their dot product per
//                        batch row, the choice per row and the vote.
// Summation orders are fixed, so the results are deterministic.

#include "kvq_internal.h"
#include "kvq_device.h"
#include "../../include/kvq.h"

namespace kvq {
namespace {

constexpr int kChunk = 64;          // tokens per workgroup of the sums kernel
constexpr int kSearchThreads = 256;

typedef __amdgpu_buffer_rsrc_t Rsrc;

// Every token row is read once: non-temporal cache policy (nt), 5% faster
// than the default policy on MI355X when the rows come from HBM.
__device__ __forceinline__ uint4 load16(Rsrc r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// NSL: 16-byte slots (8 channels) per lane, D <= 512 * NSL.
template <int NSL>
__global__ void __launch_bounds__(kSearchThreads) search_sums_kernel(const SearchParams P) {
  extern __shared__ __align__(16) float red[];     // [D]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int x = blockIdx.x, b = blockIdx.y;
  const int D = P.D;
  const int vis_chunks = P.n_windows * P.chunks_per_window;
  // this chunk's token rows
  const uint16_t* base;
  int64_t row_stride;
  int t0, t1;
  if (x < vis_chunks) {
    const int w = x / P.chunks_per_window, c = x % P.chunks_per_window;
    base = P.visual + int64_t(b) * P.visual_batch_stride;
    row_stride = P.visual_row_stride;
    t0 = w * P.S + c * kChunk;
    t1 = min(t0 + kChunk, (w + 1) * P.S);
  } else {
    base = P.text + int64_t(b) * P.text_batch_stride;
    row_stride = P.text_row_stride;
    t0 = (x - vis_chunks) * kChunk;
    t1 = min(t0 + kChunk, P.N);
  }
  float acc[NSL][8];
#pragma unroll
  for (int i = 0; i < NSL; ++i)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[i][k] = 0.f;

  const uint32_t row_bytes = uint32_t(D) * 2;
  // one row per wave at a time, the next row's loads in flight while the
  // current one is summed; rows go through range-checked resources (slots
  // past D and rows past t1 read as zero and touch no memory)
  auto load_row = [&](int t, uint4 (&v)[NSL]) {
    const int tt = t < t1 ? t : t0;      // a row of the chunk; its loads are discarded
    const Rsrc r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base + int64_t(tt) * row_stride),
                                                     short(0), int(t < t1 ? row_bytes : 0u), 0x00020000);
#pragma unroll
    for (int i = 0; i < NSL; ++i) v[i] = load16(r, uint32_t(lane + 64 * i) * 16);
  };
  uint4 cur[NSL], nxt[NSL];
  load_row(t0 + wave, cur);
  for (int t = t0 + wave; t < t1; t += 4) {
    load_row(t + 4, nxt);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NSL; ++i) {
      const uint32_t w4[4] = {cur[i].x, cur[i].y, cur[i].z, cur[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float a = h2f(w4[k] & 0xffffu), c = h2f(w4[k] >> 16);
        ss = __builtin_fmaf(a, a, ss);
        ss = __builtin_fmaf(c, c, ss);
      }
    }
    ss = wave_sum64(ss);
    // a zero row has no direction: it adds nothing
    const float inv = ss > 0.f ? 1.f / __builtin_sqrtf(ss) : 0.f;
#pragma unroll
    for (int i = 0; i < NSL; ++i) {
      const uint32_t w4[4] = {cur[i].x, cur[i].y, cur[i].z, cur[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[i][2 * k] = __builtin_fmaf(h2f(w4[k] & 0xffffu), inv, acc[i][2 * k]);
        acc[i][2 * k + 1] = __builtin_fmaf(h2f(w4[k] >> 16), inv, acc[i][2 * k + 1]);
      }
    }
#pragma unroll
    for (int i = 0; i < NSL; ++i) cur[i] = nxt[i];
  }
  // the chunk sum ((w0 + w1) + w2) + w3 of the four waves' sums: wave 0
  // stores its sum in LDS, waves 1 and 2 add theirs in turn, wave 3 adds its
  // own and writes the result (one D-float slot keeps the LDS small enough
  // for three workgroups per CU)
  float* out = P.ws + (int64_t(b) * P.n_chunks + x) * D;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int i = 0; i < NSL; ++i) {
        const int c0 = (lane + 64 * i) * 8;
        if (c0 >= D) continue;
        float4* slot = reinterpret_cast<float4*>(red + c0);
        float4 lo4 = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
        float4 hi4 = make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
        if (w > 0) {
          const float4 a = slot[0], c = slot[1];
          lo4 = make_float4(a.x + lo4.x, a.y + lo4.y, a.z + lo4.z, a.w + lo4.w);
          hi4 = make_float4(c.x + hi4.x, c.y + hi4.y, c.z + hi4.z, c.w + hi4.w);
        }
        if (w < 3) {
          slot[0] = lo4;
          slot[1] = hi4;
        } else {
          float4* dst = reinterpret_cast<float4*>(out + c0);
          dst[0] = lo4;
          dst[1] = hi4;
        }
      }
    }
    if (w < 3) __syncthreads();
  }
}

__device__ __forceinline__ float block_sum(float x, float* sh) {
  x = wave_sum64(x);
  const int wave = threadIdx.x >> 6;
  __syncthreads();                         // sh is reused across calls
  if ((threadIdx.x & 63) == 0) sh[wave] = x;
  __syncthreads();
  return ((sh[0] + sh[1]) + sh[2]) + sh[3];
}

__global__ void __launch_bounds__(kSearchThreads) search_vote_kernel(const SearchParams P) {
  __shared__ float sh[4];
  __shared__ int counts[3];                // fp16, int4, int2
  const int w = blockIdx.x;
  const int D = P.D;
  const int vis_chunks = P.n_windows * P.chunks_per_window;
  const int text_chunks = P.n_chunks - vis_chunks;
  if (threadIdx.x < 3) counts[threadIdx.x] = 0;
  const float inv_pairs = 1.f / (float(P.S) * float(P.N));
  const int D4 = D / 4;
  for (int b = 0; b < P.B; ++b) {
    const float4* part = reinterpret_cast<const float4*>(P.ws + int64_t(b) * P.n_chunks * D);
    const float4* wrow = part + int64_t(w) * P.chunks_per_window * D4;
    const float4* trow = part + int64_t(vis_chunks) * D4;
    float dot = 0.f;
    // up to four channel quads per thread (D <= 4096), all loads issued together
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = threadIdx.x + j * kSearchThreads;
      if (c >= D4) continue;
      float4 ws = make_float4(0.f, 0.f, 0.f, 0.f), ts = ws;
#pragma unroll 4
      for (int k = 0; k < P.chunks_per_window; ++k) {
        const float4 x = wrow[int64_t(k) * D4 + c];
        ws.x += x.x; ws.y += x.y; ws.z += x.z; ws.w += x.w;
      }
#pragma unroll 4
      for (int k = 0; k < text_chunks; ++k) {
        const float4 x = trow[int64_t(k) * D4 + c];
        ts.x += x.x; ts.y += x.y; ts.z += x.z; ts.w += x.w;
      }
      dot = __builtin_fmaf(ws.x, ts.x, dot);
      dot = __builtin_fmaf(ws.y, ts.y, dot);
      dot = __builtin_fmaf(ws.z, ts.z, dot);
      dot = __builtin_fmaf(ws.w, ts.w, dot);
    }
    const float score = block_sum(dot, sh) * inv_pairs;
    if (threadIdx.x == 0) {
      if (P.scores) P.scores[int64_t(b) * P.n_windows + w] = score;
      const int choice = score > P.t_high ? 0 : (score < P.t_low ? 2 : 1);
      counts[choice] += 1;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    // the most frequent width; ties to the wider one
    int best = 0;
    for (int k = 1; k < 3; ++k)
      if (counts[k] > counts[best]) best = k;
    const uint8_t bits = (w == 0 && P.first_window_fp16) ? 16 : uint8_t(best == 0 ? 16 : best == 1 ? 4 : 2);
    P.win_bits[w] = bits;
  }
}

}  // namespace

int32_t search_chunks_per_window(int32_t S) { return (S + kChunk - 1) / kChunk; }

int64_t search_chunks(int32_t n_text, int32_t n_windows, int32_t S) {
  return int64_t(n_windows) * search_chunks_per_window(S) + (n_text + kChunk - 1) / kChunk;
}

hipError_t launch_search(const SearchParams& p, hipStream_t s) {
  const int nsl = (p.D + 511) / 512;
  const size_t lds = size_t(p.D) * sizeof(float);
  const dim3 grid(unsigned(p.n_chunks), unsigned(p.B));
  switch (nsl) {
#define SEARCH_SUMS(N) \
    case N: hipLaunchKernelGGL(search_sums_kernel<N>, grid, dim3(kSearchThreads), lds, s, p); break;
    SEARCH_SUMS(1) SEARCH_SUMS(2) SEARCH_SUMS(3) SEARCH_SUMS(4)
    SEARCH_SUMS(5) SEARCH_SUMS(6) SEARCH_SUMS(7) SEARCH_SUMS(8)
#undef SEARCH_SUMS
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(search_vote_kernel, dim3(unsigned(p.n_windows)), dim3(kSearchThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvq
