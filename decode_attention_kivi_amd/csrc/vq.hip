// Decode attention over a vector-quantized (codebook) KV cache (VQ-LLM note,
// "Background" on vector quantization and the CQ-2 / CQ-4 KV-cache
// configurations): every group of 4 consecutive channels of a key or value
// is coded by an 8-bit index into its own 256-entry codebook, in R rounds
// (round r codes the residual of the rounds before it; the dequantized
// sub-vector is the sum of the R entries).  One query token per sequence and
// query head attends to all n_tok cached tokens: softmax of the scaled
// logits, then the probability-weighted sum of the dequantized values.
//
// Nothing is dequantized into memory:
//   vq_partial_kernel  grid (token chunks, B * Hkv), 4 waves; for each query
//                      head of the kv head in turn:
//                      * round by round, a table of q_g . entry for every
//                        (group, entry) in LDS (fp32, from the key codebook),
//                        so a token's logit is the sum of its R * D/4 table
//                        entries named by its codes (one 16-byte code load
//                        per 16 codes);
//                      * the chunk's softmax state (max, sum) with the
//                        probabilities kept in LDS;
//                      * the probabilities, rounded to fp16, then, round by
//                        round, the kv head's value codebook staged into the
//                        table's LDS;
//                        a lane takes 4 groups of a token (one 4-byte code
//                        load per round) and adds p times their entries into
//                        16 channel sums, which are summed over the lanes of
//                        the same groups (xor shuffles) and over the waves;
// Every sum runs in a fixed order, so the output is the same from run to run.

#include "kvq_internal.h"
#include "kvq_device.h"
#include "vq.h"

namespace kvq {
namespace {

constexpr int kVqThreads = 256;
constexpr int kVqWaves = kVqThreads / 64;

template <int D, int R>
__global__ void __launch_bounds__(kVqThreads) vq_partial_kernel(const VqParams P) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int G = D / 4;                   // channel groups (codebooks per round)
  constexpr int TB = R * G;                  // code bytes per token
  constexpr int NR = G * 256;                // codebook entries of one round
  constexpr int QPT = G / 4;                 // lanes per token in the value pass (4 groups each)
  constexpr int TPW = 64 / QPT;              // tokens per wave step in the value pass
  // region, one round at a time: the round's key table [NR] fp32 and the
  // logits [chunk] fp32 while the logits are made, then the round's value
  // codebook [NR][4] fp16 (vq_region_bytes)
  const int64_t region = vq_region_bytes(D, P.chunk_tokens);
  float* tab = reinterpret_cast<float*>(smem);
  float* xs = tab + NR;
  const uint16_t* book = reinterpret_cast<const uint16_t*>(smem);
  uint16_t* p16 = reinterpret_cast<uint16_t*>(smem + region);             // [chunk] probabilities, fp16
  float* qf = reinterpret_cast<float*>(smem + region + (int64_t(P.chunk_tokens) * 2 + 15) / 16 * 16);
  __shared__ float red[2 * kVqWaves];
  __shared__ float osum[kVqWaves][D];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int chunk = blockIdx.x;
  const int64_t stream = blockIdx.y;
  const int b = int(stream / P.Hkv), kv = int(stream % P.Hkv);
  const int t0 = chunk * P.chunk_tokens;
  const int nt = min(P.n_tok, t0 + P.chunk_tokens) - t0;   // >= 1: chunks are never empty
  const uint8_t* kc = P.k_codes + stream * P.codes_stride + int64_t(t0) * TB;
  const uint8_t* vc = P.v_codes + stream * P.codes_stride + int64_t(t0) * TB;
  const uint16_t* kb = P.k_books + int64_t(kv) * R * NR * 4;
  const uint16_t* vb = P.v_books + int64_t(kv) * R * NR * 4;

  for (int h = 0; h < P.gq; ++h) {
    const int64_t bhq = int64_t(b) * P.Hq + int64_t(kv) * P.gq + h;
    __syncthreads();                         // the previous head is done with the LDS
    for (int i = tid; i < D; i += kVqThreads) qf[i] = h2f(P.q[bhq * D + i]);
    // logits, round by round: the round's table, then its lookups added to
    // every token's logit (a token per thread, the codes of UK tokens loaded
    // together; past the end: token nt - 1, not stored)
    constexpr int UK = 4;
    float mx = -INFINITY;
    for (int r = 0; r < R; ++r) {
      __syncthreads();                       // q is in; the previous round's table is read
      const uint16_t* kbr = kb + int64_t(r) * NR * 4;
#pragma unroll 8
      for (int i = tid; i < NR; i += kVqThreads) {
        const int g = i >> 8;
        const uint2 e = *reinterpret_cast<const uint2*>(kbr + int64_t(i) * 4);
        float acc = qf[4 * g] * h2f(e.x & 0xffffu);
        acc = __builtin_fmaf(qf[4 * g + 1], h2f(e.x >> 16), acc);
        acc = __builtin_fmaf(qf[4 * g + 2], h2f(e.y & 0xffffu), acc);
        acc = __builtin_fmaf(qf[4 * g + 3], h2f(e.y >> 16), acc);
        tab[i] = acc;
      }
      __syncthreads();
      for (int tb = tid; tb < nt; tb += UK * kVqThreads) {
        uint4 u[UK][G / 16];
#pragma unroll
        for (int k = 0; k < UK; ++k) {
          const uint4* c = reinterpret_cast<const uint4*>(kc + int64_t(min(tb + k * kVqThreads, nt - 1)) * TB + r * G);
#pragma unroll
          for (int w = 0; w < G / 16; ++w) u[k][w] = c[w];
        }
#pragma unroll
        for (int k = 0; k < UK; ++k) {
          const int t = tb + k * kVqThreads;
          if (t >= nt) break;
          float acc = r == 0 ? 0.f : xs[t];
#pragma unroll
          for (int w = 0; w < G / 16; ++w) {
            const uint32_t wd[4] = {u[k][w].x, u[k][w].y, u[k][w].z, u[k][w].w};
#pragma unroll
            for (int j = 0; j < 16; ++j) acc += tab[(w * 16 + j) * 256 + ((wd[j >> 2] >> ((j & 3) * 8)) & 0xffu)];
          }
          if (r == R - 1) {
            acc *= P.scale_log2;             // base-2 logit
            mx = fmaxf(mx, acc);
          }
          xs[t] = acc;
        }
      }
    }
    mx = wave_max64(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int w = 1; w < kVqWaves; ++w) m = fmaxf(m, red[w]);
    // probabilities, rounded to fp16; the sum is of the rounded values
    float ls = 0.f;
    for (int t = tid; t < nt; t += kVqThreads) {
      const uint32_t ph = f2h(exp2f(xs[t] - m));
      p16[t] = uint16_t(ph);
      ls += h2f(ph);
    }
    ls = wave_sum64(ls);
    if (lane == 0) red[kVqWaves + wave] = ls;
    float l = 0.f;

    // o[4g + j] = sum_t p_t sum_r vbook[r][g][code_t,r,g][j], round by round
    // with the round's value codebook in the region: lane (ts, quad) takes
    // groups 4 quad .. 4 quad + 3 of tokens ts, ts + TPW * waves, ...
    const int ts = lane / QPT, quad = lane % QPT;
    float acc[4][4];
#pragma unroll
    for (int gi = 0; gi < 4; ++gi)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[gi][j] = 0.f;
    for (int r = 0; r < R; ++r) {
      __syncthreads();                       // the logits / the previous round's codebook are read
      if (r == 0) {
#pragma unroll
        for (int w = 0; w < kVqWaves; ++w) l += red[kVqWaves + w];
      }
      {
        const uint4* src = reinterpret_cast<const uint4*>(vb + int64_t(r) * NR * 4);
        uint4* dst = reinterpret_cast<uint4*>(smem);
#pragma unroll 8
        for (int i = tid; i < NR / 2; i += kVqThreads) dst[i] = src[i];
      }
      __syncthreads();
      // the codes of UV steps loaded together (past the end: token nt - 1
      // with probability 0)
      constexpr int UV = 8;
      constexpr int STEP = kVqWaves * TPW;
      for (int tb = wave * TPW + ts; tb < nt; tb += UV * STEP) {
        uint32_t c4[UV];
        float p[UV];
#pragma unroll
        for (int u = 0; u < UV; ++u) {
          const int t = tb + u * STEP;
          c4[u] = *reinterpret_cast<const uint32_t*>(vc + int64_t(min(t, nt - 1)) * TB + r * G + quad * 4);
          p[u] = t < nt ? h2f(p16[t]) : 0.f;
        }
#pragma unroll
        for (int u = 0; u < UV; ++u)
#pragma unroll
          for (int gi = 0; gi < 4; ++gi) {
            const int e = ((quad * 4 + gi) << 8) + int((c4[u] >> (8 * gi)) & 0xffu);
            const uint2 v = *reinterpret_cast<const uint2*>(book + e * 4);
            acc[gi][0] = __builtin_fmaf(p[u], h2f(v.x & 0xffffu), acc[gi][0]);
            acc[gi][1] = __builtin_fmaf(p[u], h2f(v.x >> 16), acc[gi][1]);
            acc[gi][2] = __builtin_fmaf(p[u], h2f(v.y & 0xffffu), acc[gi][2]);
            acc[gi][3] = __builtin_fmaf(p[u], h2f(v.y >> 16), acc[gi][3]);
          }
      }
    }
    // sum over the lanes of a quad (lanes quad, quad + QPT, ...), then over
    // the waves in order
#pragma unroll
    for (int gi = 0; gi < 4; ++gi)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int o = QPT; o < 64; o <<= 1) acc[gi][j] += __shfl_xor(acc[gi][j], o, 64);
    if (ts == 0) {
#pragma unroll
      for (int gi = 0; gi < 4; ++gi)
#pragma unroll
        for (int j = 0; j < 4; ++j) osum[wave][(quad * 4 + gi) * 4 + j] = acc[gi][j];
    }
    __syncthreads();
    const bool single = P.n_chunks == 1;
    float* part = P.ws + ((stream * P.n_chunks + chunk) * P.gq + h) * (D + 2);
    for (int c = tid; c < D; c += kVqThreads) {
      float o = osum[0][c];
#pragma unroll
      for (int w = 1; w < kVqWaves; ++w) o += osum[w][c];
      if (single) P.out[bhq * D + c] = o / l;
      else part[2 + c] = o;
    }
    if (!single && tid == 0) {
      part[0] = m;
      part[1] = l;
    }
  }
}

// One workgroup per (b, hq): M = the largest chunk max; chunk s weighs
// f_s = 2^(m_s - M); out = (sum_s f_s o_s) / (sum_s f_s l_s).
template <int D>
__global__ void __launch_bounds__(kVqThreads) vq_merge_kernel(const VqParams P) {
  __shared__ float f[kVqMaxChunks];
  __shared__ float red[2 * kVqWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t bhq = blockIdx.x;
  const int b = int(bhq / P.Hq), hq = int(bhq % P.Hq);
  const int64_t stream = int64_t(b) * P.Hkv + hq / P.gq;
  const int64_t step = int64_t(P.gq) * (D + 2);
  const float* w0 = P.ws + stream * P.n_chunks * step + (hq % P.gq) * (D + 2);
  const int nc = P.n_chunks;
  float mx = -INFINITY;
  for (int s = tid; s < nc; s += kVqThreads) mx = fmaxf(mx, w0[s * step]);
  mx = wave_max64(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < kVqWaves; ++w) M = fmaxf(M, red[w]);
  float lp = 0.f;
  for (int s = tid; s < nc; s += kVqThreads) {
    const float ms = w0[s * step];
    const float fs = ms == M ? 1.f : exp2f(ms - M);
    f[s] = fs;
    lp = __builtin_fmaf(w0[s * step + 1], fs, lp);
  }
  lp = wave_sum64(lp);
  if (lane == 0) red[kVqWaves + wave] = lp;
  __syncthreads();
  float L = red[kVqWaves];
#pragma unroll
  for (int w = 1; w < kVqWaves; ++w) L += red[kVqWaves + w];
  for (int c = tid; c < D; c += kVqThreads) {
    float o = 0.f;
#pragma unroll 8
    for (int s = 0; s < nc; ++s) o = __builtin_fmaf(w0[s * step + 2 + c], f[s], o);
    P.out[bhq * D + c] = o / L;
  }
}

template <int D, int R>
hipError_t launch_dr(const VqParams& p, hipStream_t s) {
  const size_t lds = size_t(vq_lds_bytes(D, p.chunk_tokens));
  hipLaunchKernelGGL((vq_partial_kernel<D, R>), dim3(unsigned(p.n_chunks), unsigned(int64_t(p.B) * p.Hkv)),
                     dim3(kVqThreads), lds, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_chunks == 1) return e;
  hipLaunchKernelGGL((vq_merge_kernel<D>), dim3(unsigned(int64_t(p.B) * p.Hq)), dim3(kVqThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

int64_t vq_lds_bytes(int D, int chunk_tokens) {
  // region, fp16 probabilities, q
  return vq_region_bytes(D, chunk_tokens) + (int64_t(chunk_tokens) * 2 + 15) / 16 * 16 + int64_t(D) * 4;
}

hipError_t launch_vq_decode(const VqParams& p, hipStream_t s) {
  if (p.D == 64) return p.R == 1 ? launch_dr<64, 1>(p, s) : launch_dr<64, 2>(p, s);
  if (p.D == 128) return p.R == 1 ? launch_dr<128, 1>(p, s) : launch_dr<128, 2>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace kvq
