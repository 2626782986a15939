// PQCache decode-time PQ search (PQCache note, "Background" on product
// quantization and "Method details", Step 4): for a query head, a table of
// q_j . centroid[j][c] per sub-space j and centroid c, then the approximate
// score of every token as the sum of the table entries its m codes name
// (the query's dot product with the key rebuilt from the centroids), then
// the Top-k tokens by score.
//
// Two kernels:
//   pq_scores_kernel  grid (token chunks, B * Hkv): the tables of the GQ query
//                     heads of one kv head in LDS (fp32 dot products of the
//                     fp16 centroids and q), then 16-byte code loads (16/m
//                     tokens per lane) and table lookups; scores fp32.
//   pq_topk_kernel    one workgroup per (b, hq): the k-th largest score is
//                     narrowed down by two levels of 2048 equal-width value
//                     buckets (histograms in LDS: the scores spread over them,
//                     where the leading bits of their float encodings would
//                     pile into a few bins and serialize the atomics), then
//                     found exactly by a radix select of the order-preserving
//                     32-bit keys of the remaining candidates; a scanned
//                     compaction writes the selected tokens in ascending
//                     order, ties at the threshold to the lower token index.

#include "kvq_internal.h"
#include "kvq_device.h"

namespace kvq {
namespace {

constexpr int kPqThreads = 256;
constexpr int kTopkThreads = 1024;

typedef __amdgpu_buffer_rsrc_t Rsrc;

// Order-preserving key of a finite float (-0 and +0 share +0's key).
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t b = __builtin_bit_cast(uint32_t, x + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <int GQ>
__global__ void __launch_bounds__(kPqThreads) pq_scores_kernel(const PqParams P) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int D = P.D, m = P.m, dm = D / m, nc = 1 << P.bits;
  const int64_t stream = blockIdx.y;
  const int b = int(stream / P.Hkv), kv = int(stream % P.Hkv);
  float* tab = reinterpret_cast<float*>(smem);                        // [GQ][m][nc]
  float* qf = tab + GQ * m * nc;                                      // [GQ][D]
  const int tid = threadIdx.x;
  const uint16_t* qg = P.q + (int64_t(b) * P.Hq + int64_t(kv) * P.gq) * D;
  for (int i = tid; i < GQ * D; i += kPqThreads) {
    const int h = i / D;
    qf[i] = h < P.gq ? h2f(qg[i]) : 0.f;
  }
  __syncthreads();
  // tables: one (j, c) per thread pass, every head at once
  const uint16_t* cen = P.centroids + stream * int64_t(m) * nc * dm;
  for (int e = tid; e < m * nc; e += kPqThreads) {
    const int j = e / nc;
    const uint4* row = reinterpret_cast<const uint4*>(cen + int64_t(e) * dm);
    float acc[GQ];
#pragma unroll
    for (int h = 0; h < GQ; ++h) acc[h] = 0.f;
    for (int k = 0; k < dm / 8; ++k) {
      const uint4 u = row[k];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float c0 = h2f(w[i] & 0xffffu), c1 = h2f(w[i] >> 16);
        const int ch = j * dm + k * 8 + 2 * i;
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
          acc[h] = __builtin_fmaf(qf[h * D + ch], c0, acc[h]);
          acc[h] = __builtin_fmaf(qf[h * D + ch + 1], c1, acc[h]);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < GQ; ++h) tab[(h * m + j) * nc + (e - j * nc)] = acc[h];
  }
  __syncthreads();
  // codes: lane loads 16 bytes = 16/m tokens; chunk = blockDim * U loads
  const int tpl = 16 / m;                                   // tokens per 16-byte load
  const int64_t t_base = int64_t(blockIdx.x) * P.chunk_tokens;
  const int64_t t_end = min(int64_t(P.n_tok), t_base + P.chunk_tokens);
  const uint8_t* cb = P.codes + stream * P.codes_stride;
  // the range check works per dword: the range is the codes rounded up to
  // 16 bytes (within the stride the caller allocated), so the last tokens'
  // codes are never cut off; bytes past n_tok * m are read and ignored
  const Rsrc rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(cb), short(0),
                                                    int((int64_t(P.n_tok) * m + 15) / 16 * 16), 0x00020000);
  for (int64_t t0 = t_base + int64_t(tid) * tpl; t0 < t_end; t0 += int64_t(kPqThreads) * tpl) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, uint32_t(t0 * m), 0, 2);
    const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
    for (int i = 0; i < tpl; ++i) {
      const int64_t t = t0 + i;
      if (t >= t_end) break;
      float s[GQ];
#pragma unroll
      for (int h = 0; h < GQ; ++h) s[h] = 0.f;
      for (int j = 0; j < m; ++j) {
        const int byte = i * m + j;
        const int code = int((w[byte >> 2] >> ((byte & 3) * 8)) & 0xffu);
#pragma unroll
        for (int h = 0; h < GQ; ++h) s[h] += tab[(h * m + j) * nc + code];
      }
#pragma unroll
      for (int h = 0; h < GQ; ++h)
        if (h < P.gq) P.scores[((int64_t(b) * P.Hq + int64_t(kv) * P.gq + h) * P.n_tok) + t] = s[h];
    }
  }
}

// Exclusive prefix sum over the block (1024 threads, 16 waves); returns this
// thread's exclusive sum and the block total in *total.
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t x, uint32_t* sh, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  if (threadIdx.x < 64) {
    uint32_t wv = threadIdx.x < kTopkThreads / 64 ? sh[threadIdx.x] : 0u;
    uint32_t wi = wv;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(wi, o, 64);
      if (lane >= o) wi += y;
    }
    if (threadIdx.x < kTopkThreads / 64) sh[32 + threadIdx.x] = wi - wv;   // exclusive wave offsets
    if (threadIdx.x == kTopkThreads / 64 - 1) sh[64] = wi;
  }
  __syncthreads();
  const uint32_t r = sh[32 + wave] + incl - x;
  *total = sh[64];
  __syncthreads();
  return r;
}

// Bucket of a score: 2^22 equal ranges of [lo, hi], taken as two levels of
// 2048 (the high 11 bits of the id are the level-1 bin, the low 11 bits the
// level-2 bin within it).  The id comes from one subtract-then-multiply, which
// leaves no multiply-add for the compiler to fuse, so every pass that
// recomputes a score's id gets the same id.  It is non-decreasing in the score
// (fp32 subtraction of a constant and multiplication by a positive constant
// preserve order), so equal scores share a bucket and a higher bucket holds
// only higher scores.
constexpr int kBins = 2048;
__device__ __forceinline__ int bucket_id(float x, float lo, float s2) {
  return min(kBins * kBins - 1, int(__fmul_rn(x - lo, s2)));
}

// The bin of hist[0..nbins) (counted from the top) that holds the k-th
// largest element: returns the bin and, in *above, the count in higher bins.
// One wave scans: lane L sums its 32 bins from the top, a wave scan finds
// the crossing lane, which walks its bins.  Caller syncs before and after.
__device__ __forceinline__ int find_bin(const uint32_t* hist, int nbins, uint32_t k, uint32_t* above,
                                        uint32_t* sh) {
  if (threadIdx.x < 64) {
    if (threadIdx.x == 0) sh[0] = sh[1] = 0;
    const int lane = threadIdx.x;
    const int per = nbins / 64;
    const int top = nbins - 1 - lane * per;             // this lane's bins: top, top-1, ..., top-per+1
    uint32_t sum = 0;
    for (int i = 0; i < per; ++i) sum += hist[top - i];
    uint32_t incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    const uint32_t excl = incl - sum;
    if (excl < k && incl >= k) {                          // exactly one lane
      uint32_t acc = excl;
      int bin = top - per + 1;
      for (int i = 0; i < per; ++i) {
        const uint32_t c = hist[top - i];
        if (acc + c >= k) { bin = top - i; break; }
        acc += c;
      }
      sh[0] = uint32_t(bin);
      sh[1] = acc;
    }
  }
  __syncthreads();
  *above = sh[1];
  return int(sh[0]);
}

__global__ void __launch_bounds__(kTopkThreads) pq_topk_kernel(const PqParams P) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t sh[72];
  __shared__ float fsh[2 * kTopkThreads / 64];
  const int64_t head = blockIdx.x;                            // b * Hq + hq
  const float* sc = P.scores + head * P.n_tok;
  const int n = P.n_tok, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // range of the scores
  float lo = INFINITY, hi = -INFINITY;
  for (int t = tid; t < n; t += kTopkThreads) {
    const float x = sc[t] + 0.0f;
    lo = fminf(lo, x);
    hi = fmaxf(hi, x);
  }
  lo = span_min<64>(lo);
  hi = span_max<64>(hi);
  if (lane == 0) { fsh[wave] = lo; fsh[16 + wave] = hi; }
  __syncthreads();
  lo = fsh[0];
  hi = fsh[16];
  for (int w = 1; w < kTopkThreads / 64; ++w) { lo = fminf(lo, fsh[w]); hi = fmaxf(hi, fsh[16 + w]); }
  // one bucket when the range is empty (or too narrow for a finite scale):
  // the radix passes then resolve everything
  float s2 = hi > lo ? float(kBins * kBins) / (hi - lo) : 0.f;
  if (!(s2 < 1e30f)) s2 = 0.f;

  // level 1 and level 2 buckets narrow the k-th largest score down
  uint32_t k_rem = uint32_t(P.top_k), above;
  for (int i = tid; i < kBins; i += kTopkThreads) hist[i] = 0;
  __syncthreads();
  for (int t = tid; t < n; t += kTopkThreads) atomicAdd(&hist[bucket_id(sc[t] + 0.0f, lo, s2) >> 11], 1u);
  __syncthreads();
  const int b1 = find_bin(hist, kBins, k_rem, &above, sh);
  k_rem -= above;
  __syncthreads();
  for (int i = tid; i < kBins; i += kTopkThreads) hist[i] = 0;
  __syncthreads();
  for (int t = tid; t < n; t += kTopkThreads) {
    const int id = bucket_id(sc[t] + 0.0f, lo, s2);
    if ((id >> 11) == b1) atomicAdd(&hist[id & (kBins - 1)], 1u);
  }
  __syncthreads();
  const int b2 = find_bin(hist, kBins, k_rem, &above, sh);
  k_rem -= above;
  __syncthreads();

  // exact key among the candidates of bucket (b1, b2): four radix passes of
  // 8 bits over their order-preserving keys
  uint32_t prefix = 0, mask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    for (int t = tid; t < n; t += kTopkThreads) {
      const float x = sc[t] + 0.0f;
      if (bucket_id(x, lo, s2) != b1 * kBins + b2) continue;
      const uint32_t key = order_key(x);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xffu], 1u);
    }
    __syncthreads();
    const int d = find_bin(hist, 256, k_rem, &above, sh);
    k_rem -= above;
    prefix |= uint32_t(d) << shift;
    mask |= 0xffu << shift;
    __syncthreads();
  }
  // prefix is the threshold key T: every key > T is selected and the first
  // k_rem keys == T by token index
  const uint32_t T = prefix;
  const int seg = (n + kTopkThreads - 1) / kTopkThreads;
  const int t0 = min(n, tid * seg), t1 = min(n, t0 + seg);
  uint32_t gt = 0, eq = 0;
  for (int t = t0; t < t1; ++t) {
    const uint32_t key = order_key(sc[t]);
    gt += key > T;
    eq += key == T;
  }
  uint32_t tot;
  const uint32_t gt_before = block_exclusive_sum(gt, sh, &tot);
  const uint32_t eq_before = block_exclusive_sum(eq, sh, &tot);
  uint32_t pos = gt_before + min(eq_before, k_rem);
  uint32_t eq_seen = eq_before;
  int32_t* out = P.top_idx + head * P.top_k;
  for (int t = t0; t < t1; ++t) {
    const uint32_t key = order_key(sc[t]);
    if (key > T) {
      out[pos++] = t;
    } else if (key == T) {
      if (eq_seen < k_rem) out[pos++] = t;
      ++eq_seen;
    }
  }
}

}  // namespace

int64_t pq_scores_lds_bytes(int gq_pow2, int D, int m, int bits) {
  return int64_t(gq_pow2) * m * (int64_t(1) << bits) * 4 + int64_t(gq_pow2) * D * 4;
}

hipError_t launch_pq_search(const PqParams& p, int GQ, hipStream_t s) {
  const int64_t chunks = (int64_t(p.n_tok) + p.chunk_tokens - 1) / p.chunk_tokens;
  const dim3 grid(unsigned(chunks), unsigned(int64_t(p.B) * p.Hkv));
  const size_t lds = size_t(pq_scores_lds_bytes(GQ, p.D, p.m, p.bits));
  switch (GQ) {
    case 1: hipLaunchKernelGGL((pq_scores_kernel<1>), grid, dim3(kPqThreads), lds, s, p); break;
    case 2: hipLaunchKernelGGL((pq_scores_kernel<2>), grid, dim3(kPqThreads), lds, s, p); break;
    case 4: hipLaunchKernelGGL((pq_scores_kernel<4>), grid, dim3(kPqThreads), lds, s, p); break;
    case 8: hipLaunchKernelGGL((pq_scores_kernel<8>), grid, dim3(kPqThreads), lds, s, p); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pq_topk_kernel, dim3(unsigned(int64_t(p.B) * p.Hq)), dim3(kTopkThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvq
