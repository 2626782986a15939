// PQCache decode-time PQ search (PQCache note, "Background" on product
// quantization and "Method details", Step 4): for a query head, a table of
// q_j . centroid[j][c] per sub-space j and centroid c, then the approximate
// score of every token as the sum of the table entries its m codes name
// (the query's dot product with the key rebuilt from the centroids), then
// the Top-k tokens by score.
//
// Three kernels:
//   pq_scores_kernel  grid (token chunks, B * Hkv, head blocks of up to 8
//                     query heads): the tables of a head block of one kv head in LDS (fp32 dot products of the
//                     fp16 centroids and q), then a token per lane (its m
//                     code bytes in one load) and table lookups; scores fp32,
//                     stored by consecutive lanes to consecutive tokens.
//   pq_topk_kernel    one workgroup per (b, hq): the k-th largest score is
//                     narrowed down by two levels of 2048 equal-width value
//                     buckets (histograms in LDS: the scores spread over them,
//                     where the leading bits of their float encodings would
//                     pile into a few bins and serialize the atomics), then
//                     found exactly by a radix select of the order-preserving
//                     32-bit keys of the remaining candidates; a ballot-based
//                     compaction writes the selected tokens in ascending
//                     order, ties at the threshold to the lower token index.
//   pq_fused_kernel   one workgroup per (b, hq) doing both, the head's scores
//                     resident in LDS (contexts up to about 38K tokens).

#include "kvq_internal.h"
#include "pq.h"
#include "kvq_device.h"

namespace kvq {
namespace {

// threads of a scores workgroup: one round of token loads covers a 4096-token
// chunk, and the tables take a fraction of an entry per thread; 512 where the
// tables of 8 heads x 16 sub-spaces need more than 128 registers a lane
__host__ __device__ constexpr int pq_scores_threads(int GQ, int M) { return GQ * M >= 128 ? 512 : 1024; }
constexpr int kTopkThreads = 1024;

typedef __amdgpu_buffer_rsrc_t Rsrc;

// Order-preserving key of a finite float (-0 and +0 share +0's key).
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t b = __builtin_bit_cast(uint32_t, x + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <int GQ, int M>
__global__ void __launch_bounds__(pq_scores_threads(GQ, M)) pq_scores_kernel(const PqParams P) {
  constexpr int kPqThreads = pq_scores_threads(GQ, M);
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int m = M;
  const int D = P.D, dm = D / m, nc = 1 << P.bits;
  const int64_t stream = blockIdx.y;
  const int b = int(stream / P.Hkv), kv = int(stream % P.Hkv);
  float* tab = reinterpret_cast<float*>(smem);                        // [GQ][m][nc]
  float* qf = tab + GQ * m * nc;                                      // [GQ][D]
  const int tid = threadIdx.x;
  // query heads h0 .. h0 + nh - 1 of the kv head (head block blockIdx.z)
  const int h0 = int(blockIdx.z) * GQ;
  const int nh = min(GQ, P.gq - h0);
  const uint16_t* qg = P.q + (int64_t(b) * P.Hq + int64_t(kv) * P.gq + h0) * D;
  for (int i = tid; i < GQ * D; i += kPqThreads) {
    const int h = i / D;
    qf[i] = h < nh ? h2f(qg[i]) : 0.f;
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
  // one token per lane (its m code bytes), UT tokens in flight, so that
  // consecutive lanes store consecutive scores; past the end: token
  // t_end - 1, not stored; only the low `bits` bits of a code byte index
  // the table
  constexpr int UT = 4;
  constexpr int NW = (M + 3) / 4;                           // code words per token
  const int64_t t_base = int64_t(blockIdx.x) * P.chunk_tokens;
  const int64_t t_end = min(int64_t(P.n_tok), t_base + P.chunk_tokens);
  const uint8_t* cb = P.codes + stream * P.codes_stride;
  const uint32_t cmask = uint32_t(nc - 1);
  float* out0 = P.scores + (int64_t(b) * P.Hq + int64_t(kv) * P.gq + h0) * P.n_tok;
  for (int64_t tb = t_base + tid; tb < t_end; tb += UT * kPqThreads) {
    uint32_t w[UT][NW];
#pragma unroll
    for (int u = 0; u < UT; ++u) {
      const int64_t t = min(tb + u * kPqThreads, t_end - 1);
      if constexpr (M == 1) {
        w[u][0] = cb[t];
      } else if constexpr (M == 2) {
        w[u][0] = reinterpret_cast<const uint16_t*>(cb)[t];
      } else if constexpr (M == 4) {
        w[u][0] = reinterpret_cast<const uint32_t*>(cb)[t];
      } else if constexpr (M == 8) {
        const uint2 x = reinterpret_cast<const uint2*>(cb)[t];
        w[u][0] = x.x;
        w[u][1] = x.y;
      } else {
        const uint4 x = reinterpret_cast<const uint4*>(cb)[t];
        w[u][0] = x.x;
        w[u][1] = x.y;
        w[u][2] = x.z;
        w[u][3] = x.w;
      }
    }
#pragma unroll
    for (int u = 0; u < UT; ++u) {
      const int64_t t = tb + u * kPqThreads;
      if (t >= t_end) break;
      float sc[GQ];
#pragma unroll
      for (int h = 0; h < GQ; ++h) sc[h] = 0.f;
#pragma unroll
      for (int j = 0; j < M; ++j) {
        const int code = int((w[u][j >> 2] >> ((j & 3) * 8)) & cmask);
#pragma unroll
        for (int h = 0; h < GQ; ++h) sc[h] += tab[(h * M + j) * nc + code];
      }
#pragma unroll
      for (int h = 0; h < GQ; ++h)
        if (h < nh) out0[int64_t(h) * P.n_tok + t] = sc[h];
    }
  }
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
  return min(kBins * kBins - 1, max(0, int(__fmul_rn(x - lo, s2))));
}

// Scale of bucket_id for the range [lo, hi]: one bucket when the range is
// empty (or too narrow for a finite scale); the radix passes then resolve
// everything.
__device__ __forceinline__ float bucket_scale(float lo, float hi) {
  const float s2 = hi > lo ? float(kBins * kBins) / (hi - lo) : 0.f;
  return s2 < 1e30f ? s2 : 0.f;
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

// f(t, sc[t]) for every t < n, the block's threads striding over the
// tokens with U reads in flight per thread (4 from LDS, 16 from memory,
// where the latency is longer).  Reads past the end take sc[n - 1]
// (n >= 1) and are not passed on: unconditional reads issue back to back.
// With V4 (n a multiple of 4, sc 16-byte aligned) a read is 4 consecutive
// tokens, so four times the bytes are in flight.
template <int U = 4, bool V4 = false, typename F>
__device__ __forceinline__ void for_scores(const float* sc, int n, F&& f) {
  if constexpr (V4) {
    const float4* s4 = reinterpret_cast<const float4*>(sc);
    for (int t0 = 4 * int(threadIdx.x); t0 < n; t0 += 4 * U * kTopkThreads) {
      float4 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = s4[min(t0 + 4 * u * kTopkThreads, n - 4) >> 2];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = t0 + 4 * u * kTopkThreads;
        if (t < n) {
          f(t, x[u].x + 0.0f);
          f(t + 1, x[u].y + 0.0f);
          f(t + 2, x[u].z + 0.0f);
          f(t + 3, x[u].w + 0.0f);
        }
      }
    }
  } else {
    for (int t0 = threadIdx.x; t0 < n; t0 += U * kTopkThreads) {
      float x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = sc[min(t0 + u * kTopkThreads, n - 1)];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (t0 + u * kTopkThreads < n) f(t0 + u * kTopkThreads, x[u] + 0.0f);
    }
  }
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u));
}

// f(t, sc[t]) for every t of one wave's segment [w0, w1) of the scores, the
// wave's lanes on consecutive tokens with U reads in flight per lane; with
// V4 (w0 and w1 multiples of 4) a read is 4 consecutive tokens.
template <int U, bool V4, typename F>
__device__ __forceinline__ void for_segment(const float* sc, int n, int w0, int w1, F&& f) {
  const int lane = threadIdx.x & 63;
  if constexpr (V4) {
    const float4* s4 = reinterpret_cast<const float4*>(sc);
    for (int t0 = w0; t0 < w1; t0 += 256 * U) {
      float4 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = s4[min(t0 + u * 256 + 4 * lane, n - 4) >> 2];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = t0 + u * 256 + 4 * lane;
        if (t < w1) {
          f(t, x[u].x + 0.0f);
          f(t + 1, x[u].y + 0.0f);
          f(t + 2, x[u].z + 0.0f);
          f(t + 3, x[u].w + 0.0f);
        }
      }
    }
  } else {
    for (int t0 = w0; t0 < w1; t0 += 64 * U) {
      float x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = sc[min(t0 + u * 64 + lane, n - 1)];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (t0 + u * 64 + lane < w1) f(t0 + u * 64 + lane, x[u] + 0.0f);
    }
  }
}

// Candidates of the threshold's bucket kept as a list of keys (in hist past
// the 256 radix counters), each with the segment (wave) of its token in a
// byte array after the keys, when they are few; more (many equal scores)
// fall back to radix passes and a counting pass over all n scores.
constexpr int kCand = 1408;
static_assert(kCand * 5 <= (kBins - 256) * 4, "keys and segment bytes fit in hist");

// The k largest of sc[0..n) (LDS or global memory, every score within
// [lo, hi]) into out[0..k) in ascending token order, ties at the threshold to
// the lower token index.  copy (may be null) receives sc[0..n).  hist holds
// kBins counters: with l1_ready the caller has filled it with the level-1
// histogram (bucket_id(x, lo, bucket_scale(lo, hi)) >> 11 of every score)
// and synced.  Every thread of the block calls.
template <int U, bool V4 = false>
__device__ __forceinline__ void select_top_k(const float* sc, int n, uint32_t k, float lo, float hi,
                                             int32_t* out, float* copy, uint32_t* hist, uint32_t* sh,
                                             bool l1_ready) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float s2 = bucket_scale(lo, hi);
  // wave w owns the contiguous segment [w0, w1) of the tokens in the
  // candidate pass and the compaction
  constexpr int NW = kTopkThreads / 64;
  constexpr int kSegAlign = V4 ? 256 : 64;
  const int seg = ((n + NW - 1) / NW + kSegAlign - 1) / kSegAlign * kSegAlign;
  const int w0 = min(n, wave * seg), w1 = min(n, w0 + seg);

  // level 1 and level 2 buckets narrow the k-th largest score down
  uint32_t k_rem = k, above;
  if (!l1_ready) {
    for (int i = tid; i < kBins; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    for_scores<U, V4>(sc, n, [&](int t, float x) { atomicAdd(&hist[bucket_id(x, lo, s2) >> 11], 1u); });
    __syncthreads();
  }
  const int b1 = find_bin(hist, kBins, k_rem, &above, sh);
  const uint32_t in_b1 = hist[b1];
  k_rem -= above;
  __syncthreads();
  // candidates: the members of bucket b1 when they fit the list, else of the
  // level-2 bucket (b1, b2) within it; a candidate has id >> cshift == target
  int target = b1, cshift = 11;
  if (in_b1 > uint32_t(kCand)) {
    for (int i = tid; i < kBins; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    for_scores<U, V4>(sc, n, [&](int t, float x) {
      const int id = bucket_id(x, lo, s2);
      if ((id >> 11) == b1) atomicAdd(&hist[id & (kBins - 1)], 1u);
    });
    __syncthreads();
    const int b2 = find_bin(hist, kBins, k_rem, &above, sh);
    k_rem -= above;
    target = b1 * kBins + b2;
    cshift = 0;
  }
  if (tid == 0) sh[70] = 0;
  __syncthreads();
  // candidate pass over the wave's segment, which also counts the segment's
  // tokens in higher buckets (bucket ids are non-decreasing in the score:
  // those scores exceed every candidate's, the lower buckets' are below)
  uint32_t* cand = hist + 256;
  uint8_t* cseg = reinterpret_cast<uint8_t*>(cand + kCand);
  uint32_t gt_b = 0;
  for_segment<U, V4>(sc, n, w0, w1, [&](int t, float x) {
    if (copy) copy[t] = x;
    const int c = bucket_id(x, lo, s2) >> cshift;
    gt_b += c > target;
    if (c == target) {
      const uint32_t slot = atomicAdd(&sh[70], 1u);
      if (slot < uint32_t(kCand)) {
        cand[slot] = order_key(x);
        cseg[slot] = uint8_t(wave);
      }
    }
  });
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) gt_b += __shfl_xor(gt_b, o, 64);
  if (lane == 0) {
    sh[32 + wave] = gt_b;
    sh[48 + wave] = 0;
  }
  __syncthreads();
  const uint32_t n_cand = sh[70];
  __syncthreads();

  // exact key among the candidates: four radix passes of 8 bits over their
  // order-preserving keys
  uint32_t prefix = 0, mask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    if (n_cand <= uint32_t(kCand)) {
      for (int i = tid; i < int(n_cand); i += kTopkThreads) {
        const uint32_t key = cand[i];
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xffu], 1u);
      }
    } else {
      for_scores<U, V4>(sc, n, [&](int t, float x) {
        if ((bucket_id(x, lo, s2) >> cshift) != target) return;
        const uint32_t key = order_key(x);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xffu], 1u);
      });
    }
    __syncthreads();
    const int d = find_bin(hist, 256, k_rem, &above, sh);
    k_rem -= above;
    prefix |= uint32_t(d) << shift;
    mask |= 0xffu << shift;
    __syncthreads();
  }

  // prefix is the threshold key T of score Tf: every score > Tf is selected
  // and the first k_rem scores == Tf by token index (float comparisons agree
  // with the key order, -0 == +0 included).  Compaction: per segment the
  // greater and equal scores are counted (from the candidate list, or by a
  // pass of ballots when it overflowed), the segment totals are scanned, and
  // a pass writes each selected token to the greater tokens before it plus
  // the selected equal tokens before it.
  const float Tf = __builtin_bit_cast(float, (prefix & 0x80000000u) ? (prefix & 0x7fffffffu) : ~prefix);
  if (n_cand <= uint32_t(kCand)) {
    for (int i = tid; i < int(n_cand); i += kTopkThreads) {
      const uint32_t key = cand[i];
      if (key >= prefix) atomicAdd(&sh[(key > prefix ? 32 : 48) + cseg[i]], 1u);
    }
  } else {
    uint32_t gt_w = 0, eq_w = 0;
    if constexpr (V4) {
      const float4* s4 = reinterpret_cast<const float4*>(sc);
      for (int t0 = w0; t0 < w1; t0 += 256 * U) {
        float4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = s4[min(t0 + u * 256 + 4 * lane, n - 4) >> 2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int tb = t0 + u * 256 + 4 * lane;
          const float xs[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool in = tb + j < w1;
            gt_w += uint32_t(__popcll(__ballot(in && xs[j] > Tf)));
            eq_w += uint32_t(__popcll(__ballot(in && xs[j] == Tf)));
          }
        }
      }
    } else {
      for (int t0 = w0; t0 < w1; t0 += 64 * U) {
        float x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = sc[min(t0 + u * 64 + lane, n - 1)];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const bool in = t0 + u * 64 + lane < w1;
          gt_w += uint32_t(__popcll(__ballot(in && x[u] > Tf)));
          eq_w += uint32_t(__popcll(__ballot(in && x[u] == Tf)));
        }
      }
    }
    if (lane == 0) {
      sh[32 + wave] = gt_w;
      sh[48 + wave] = eq_w;
    }
  }
  __syncthreads();
  uint32_t gb = 0, eb = 0;
  for (int w = 0; w < wave; ++w) {
    gb += sh[32 + w];
    eb += sh[48 + w];
  }
  if constexpr (V4) {
    // 4 consecutive tokens per lane per read: lane L's token j of a step
    // follows every token of the lower lanes and its own tokens before j
    const float4* s4 = reinterpret_cast<const float4*>(sc);
    for (int t0 = w0; t0 < w1; t0 += 256 * U) {
      float4 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = s4[min(t0 + u * 256 + 4 * lane, n - 4) >> 2];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int tb = t0 + u * 256 + 4 * lane;
        const float xs[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
        bool g[4], e[4];
        uint64_t mg[4], me[4];
        uint32_t g_low = 0, e_low = 0;            // selected tokens of the lower lanes
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          g[j] = tb + j < w1 && xs[j] > Tf;
          e[j] = tb + j < w1 && xs[j] == Tf;
          mg[j] = __ballot(g[j]);
          me[j] = __ballot(e[j]);
          g_low += lanes_below(mg[j]);
          e_low += lanes_below(me[j]);
        }
        uint32_t g_own = 0, e_own = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t g_before = gb + g_low + g_own, e_before = eb + e_low + e_own;
          if (g[j]) out[g_before + min(e_before, k_rem)] = tb + j;
          else if (e[j] && e_before < k_rem) out[g_before + e_before] = tb + j;
          g_own += g[j];
          e_own += e[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          gb += uint32_t(__popcll(mg[j]));
          eb += uint32_t(__popcll(me[j]));
        }
      }
    }
  } else {
    for (int t0 = w0; t0 < w1; t0 += 64 * U) {
      float x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = sc[min(t0 + u * 64 + lane, n - 1)];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = t0 + u * 64 + lane;
        const bool gt = t < w1 && x[u] > Tf, eq = t < w1 && x[u] == Tf;
        const uint64_t mg = __ballot(gt), me = __ballot(eq);
        const uint32_t g_before = gb + lanes_below(mg), e_before = eb + lanes_below(me);
        if (gt) out[g_before + min(e_before, k_rem)] = t;
        else if (eq && e_before < k_rem) out[g_before + e_before] = t;
        gb += uint32_t(__popcll(mg));
        eb += uint32_t(__popcll(me));
      }
    }
  }
}

// Top-k of the scores pq_scores_kernel wrote: one workgroup per (b, hq).
// The score range comes from the head's tables (per sub-space the least and
// greatest q_j . centroid, summed) instead of a pass over the scores: bucket
// ids are clamped and non-decreasing, so a bound that a rounding difference
// leaves a score just outside only widens the end buckets.
__global__ void __launch_bounds__(kTopkThreads) pq_topk_kernel(const PqParams P) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t sh[72];
  __shared__ float fsh[2 * kTopkThreads / 64];
  __shared__ float tabr[16 * 256];                           // [m][2^bits] table entries
  const int64_t head = blockIdx.x;                            // b * Hq + hq
  const int b = int(head / P.Hq), hq = int(head % P.Hq);
  const int D = P.D, m = P.m, dm = D / m, nc = 1 << P.bits;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint16_t* qh = P.q + head * D;
  const uint16_t* cen = P.centroids + (int64_t(b) * P.Hkv + hq / P.gq) * int64_t(m) * nc * dm;
  for (int e = tid; e < m * nc; e += kTopkThreads) {
    const int j = e / nc;
    const uint4* row = reinterpret_cast<const uint4*>(cen + int64_t(e) * dm);
    float acc = 0.f;
    for (int kk = 0; kk < dm / 8; ++kk) {
      const uint4 u = row[kk];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc = __builtin_fmaf(h2f(qh[j * dm + kk * 8 + 2 * i]), h2f(w[i] & 0xffffu), acc);
        acc = __builtin_fmaf(h2f(qh[j * dm + kk * 8 + 2 * i + 1]), h2f(w[i] >> 16), acc);
      }
    }
    tabr[e] = acc;
  }
  __syncthreads();
  if (wave < m) {
    float a = INFINITY, z = -INFINITY;
    for (int c = lane; c < nc; c += 64) {
      a = fminf(a, tabr[wave * nc + c]);
      z = fmaxf(z, tabr[wave * nc + c]);
    }
    a = span_min<64>(a);
    z = span_max<64>(z);
    if (lane == 0) { fsh[wave] = a; fsh[16 + wave] = z; }
  }
  __syncthreads();
  float lo = 0.f, hi = 0.f;
  for (int j = 0; j < m; ++j) {
    lo += fsh[j];
    hi += fsh[16 + j];
  }
  // 16-byte reads when every head's scores start 16-byte aligned
  const float* sc = P.scores + head * P.n_tok;
  if ((P.n_tok & 3) == 0)
    select_top_k<16, true>(sc, P.n_tok, uint32_t(P.top_k), lo, hi, P.top_idx + head * P.top_k, nullptr, hist, sh,
                           false);
  else
    select_top_k<16, false>(sc, P.n_tok, uint32_t(P.top_k), lo, hi, P.top_idx + head * P.top_k, nullptr, hist, sh,
                            false);
}

// Whole search of one (b, hq) with its scores resident in LDS: the head's
// table, a bound on the score range from it, the scores of all n_tok tokens
// from the codes with their level-1 histogram, then the rest of the Top-k
// from LDS; the scores are also written out.  D = head dim, M = sub-spaces
// (1, 2, 4, 8, 16).  Dynamic LDS: scores [round16(n_tok)] | table
// [M][2^bits] | q [D], fp32.
template <int D, int M>
__global__ void __launch_bounds__(kTopkThreads) pq_fused_kernel(const PqParams P) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t sh[72];
  __shared__ float fsh[2 * kTopkThreads / 64];
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int TPL = 16 / M;                                  // tokens per 16-byte code load
  constexpr int U = 4;                                          // code loads in flight per lane
  constexpr int dm = D / M;
  const int nc = 1 << P.bits, n = P.n_tok, tid = threadIdx.x;
  const int64_t head = blockIdx.x;                              // b * Hq + hq
  const int b = int(head / P.Hq), hq = int(head % P.Hq);
  const int64_t stream = int64_t(b) * P.Hkv + hq / P.gq;
  float* ssc = reinterpret_cast<float*>(smem);
  float* tab = ssc + (n + 15) / 16 * 16;
  float* qf = tab + M * nc;
  for (int i = tid; i < D; i += kTopkThreads) qf[i] = h2f(P.q[head * D + i]);
  __syncthreads();
  // table: q_j . centroid[j][c], one (j, c) per thread pass
  const uint16_t* cen = P.centroids + stream * int64_t(M) * nc * dm;
  for (int e = tid; e < M * nc; e += kTopkThreads) {
    const int j = e / nc;
    const uint4* row = reinterpret_cast<const uint4*>(cen + int64_t(e) * dm);
    const float* qj = qf + j * dm;
    uint4 rv[dm / 8];
#pragma unroll
    for (int kk = 0; kk < dm / 8; ++kk) rv[kk] = row[kk];
    float acc = 0.f;
#pragma unroll
    for (int kk = 0; kk < dm / 8; ++kk) {
      const uint4 u = rv[kk];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc = __builtin_fmaf(qj[kk * 8 + 2 * i], h2f(w[i] & 0xffffu), acc);
        acc = __builtin_fmaf(qj[kk * 8 + 2 * i + 1], h2f(w[i] >> 16), acc);
      }
    }
    tab[e] = acc;
  }
  __syncthreads();
  // range of the scores before any is computed: per sub-space the least and
  // greatest table entry, summed in the order the scores are (rounded fp32
  // addition is monotone, so every score lies within it)
  const int lane = tid & 63, wave = tid >> 6;
  if (wave < M) {
    float a = INFINITY, z = -INFINITY;
    for (int c = lane; c < nc; c += 64) {
      a = fminf(a, tab[wave * nc + c]);
      z = fmaxf(z, tab[wave * nc + c]);
    }
    a = span_min<64>(a);
    z = span_max<64>(z);
    if (lane == 0) { fsh[wave] = a; fsh[16 + wave] = z; }
  }
  for (int i = tid; i < kBins; i += kTopkThreads) hist[i] = 0;
  __syncthreads();
  float lo = 0.f, hi = 0.f;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    lo += fsh[j];
    hi += fsh[16 + j];
  }
  const float s2 = bucket_scale(lo, hi);
  // scores and their level-1 histogram: U 16-byte code loads per lane in
  // flight; loads past the codes' range (round16(n_tok * M) bytes) return
  // zeros and their tokens are neither stored nor counted; only the low
  // `bits` bits of a code byte index the table
  const Rsrc rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(P.codes + stream * P.codes_stride),
                                                    short(0), int((int64_t(n) * M + 15) / 16 * 16), 0x00020000);
  const uint32_t cmask = uint32_t(nc - 1);
  for (int base = tid * TPL; base < n; base += U * kTopkThreads * TPL) {
    uint32_t w[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, uint32_t(base + u * kTopkThreads * TPL) * M, 0, 2);
      w[u][0] = v[0]; w[u][1] = v[1]; w[u][2] = v[2]; w[u][3] = v[3];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t0 = base + u * kTopkThreads * TPL;
      if (t0 >= n) break;
      float s[TPL];
#pragma unroll
      for (int i = 0; i < TPL; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < M; ++j) {
          const int byte = i * M + j;
          acc += tab[j * nc + ((w[u][byte >> 2] >> ((byte & 3) * 8)) & cmask)];
        }
        s[i] = acc;
        if (t0 + i < n) atomicAdd(&hist[bucket_id(acc + 0.0f, lo, s2) >> 11], 1u);
      }
      if constexpr (TPL >= 4) {
#pragma unroll
        for (int i = 0; i < TPL; i += 4)
          *reinterpret_cast<float4*>(ssc + t0 + i) = make_float4(s[i], s[i + 1], s[i + 2], s[i + 3]);
      } else if constexpr (TPL == 2) {
        *reinterpret_cast<float2*>(ssc + t0) = make_float2(s[0], s[1]);
      } else {
        ssc[t0] = s[0];
      }
    }
  }
  __syncthreads();
  select_top_k<4>(ssc, n, uint32_t(P.top_k), lo, hi, P.top_idx + head * P.top_k, P.scores + head * n, hist, sh,
                  true);
}

}  // namespace

int64_t pq_fused_lds_bytes(int n_tok, int D, int m, int bits) {
  // dynamic part plus the kernel's static arrays (hist, sh, fsh)
  return (int64_t(n_tok + 15) / 16 * 16 + int64_t(m) * (int64_t(1) << bits) + D) * 4 +
         (kBins + 72 + 2 * kTopkThreads / 64) * 4;
}

int64_t pq_scores_lds_bytes(int gq_pow2, int D, int m, int bits) {
  return int64_t(gq_pow2) * m * (int64_t(1) << bits) * 4 + int64_t(gq_pow2) * D * 4;
}

hipError_t launch_pq_search(const PqParams& p, int GQ, bool fused, hipStream_t s) {
  if (fused) {
    const dim3 grid(unsigned(int64_t(p.B) * p.Hq));
    const size_t lds = size_t(pq_fused_lds_bytes(p.n_tok, p.D, p.m, p.bits)) - (kBins + 72 + 2 * kTopkThreads / 64) * 4;
#define PQ_FUSED(D_, M_) hipLaunchKernelGGL((pq_fused_kernel<D_, M_>), grid, dim3(kTopkThreads), lds, s, p)
    if (p.D == 64) {
      switch (p.m) {
        case 1: PQ_FUSED(64, 1); break;
        case 2: PQ_FUSED(64, 2); break;
        case 4: PQ_FUSED(64, 4); break;
        case 8: PQ_FUSED(64, 8); break;
        default: return hipErrorInvalidValue;
      }
    } else if (p.D == 128) {
      switch (p.m) {
        case 1: PQ_FUSED(128, 1); break;
        case 2: PQ_FUSED(128, 2); break;
        case 4: PQ_FUSED(128, 4); break;
        case 8: PQ_FUSED(128, 8); break;
        case 16: PQ_FUSED(128, 16); break;
        default: return hipErrorInvalidValue;
      }
    } else {
      return hipErrorInvalidValue;
    }
#undef PQ_FUSED
    return hipGetLastError();
  }
  const int64_t chunks = (int64_t(p.n_tok) + p.chunk_tokens - 1) / p.chunk_tokens;
  const dim3 grid(unsigned(chunks), unsigned(int64_t(p.B) * p.Hkv), unsigned((p.gq + GQ - 1) / GQ));
  const size_t lds = size_t(pq_scores_lds_bytes(GQ, p.D, p.m, p.bits));
#define PQ_SCORES(G_, M_) \
  hipLaunchKernelGGL((pq_scores_kernel<G_, M_>), grid, dim3(pq_scores_threads(G_, M_)), lds, s, p)
#define PQ_SCORES_M(G_)                      \
  switch (p.m) {                             \
    case 1: PQ_SCORES(G_, 1); break;         \
    case 2: PQ_SCORES(G_, 2); break;         \
    case 4: PQ_SCORES(G_, 4); break;         \
    case 8: PQ_SCORES(G_, 8); break;         \
    case 16: PQ_SCORES(G_, 16); break;       \
    default: return hipErrorInvalidValue;    \
  }
  switch (GQ) {
    case 1: PQ_SCORES_M(1); break;
    case 2: PQ_SCORES_M(2); break;
    case 4: PQ_SCORES_M(4); break;
    case 8: PQ_SCORES_M(8); break;
    default: return hipErrorInvalidValue;
  }
#undef PQ_SCORES_M
#undef PQ_SCORES
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pq_topk_kernel, dim3(unsigned(int64_t(p.B) * p.Hq)), dim3(kTopkThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvq
