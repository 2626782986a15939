// Decode-step attention over a low-bit quantized KV cache, split over the
// context (FlashDecoding dataflow, as the VQ-LLM note's reference [10]
// describes) with a final cross-split softmax merge.
//
// Per workgroup: one cache stream (batch b, kv head h), the GQ query heads
// that share it, and a range of tokens whose keys come from one source (a
// quantized run or the fp16 residual) and whose values come from one source.
//   1. q*s per key group and channel (fp16 pairs) and the group's bias
//      sum_c q_c z_c are staged in LDS (per-channel key scales: KIVI note,
//      "Method details");
//   2. logits: 16-byte loads of packed codes, in-register unpack of code
//      pairs into fp16 (offset + code), v_dot2_f32_f16 against q*s; the
//      residual part is q . K_r over fp16 rows (A = Concat([A_g, A_r]));
//   3. the split's max and sum of exp2(logit - max), one softmax over the
//      concatenation (KIVI Algorithm 1; WindowQuant Sec. 3.3.1);
//   4. A.V: value codes are stored as token pairs, so one fp16 pair holds the
//      same channel of two tokens and v_dot2 accumulates p*s over two tokens
//      per instruction; the per-token zero points are summed separately;
//   5. partial (max, sum, o[d]) per query head go to the workspace; the merge
//      kernel rescales and adds them.
// Logits are kept in base 2 (q is pre-scaled by sm_scale * log2 e).

#include "kvq_internal.h"
#include "kvq_device.h"

namespace kvq {
namespace {

constexpr int NT = kThreads;
constexpr int U = 2;   // 16-byte loads in flight per thread

struct Lds {
  float* qf;        // [GQ][D]     q * scale_log2 (fp32)
  uint32_t* qh;     // [GQ][D/2]   q as fp16 pairs
  uint32_t* qs;     // [NGMAX][GQ][D/2]  fp16(q*s) pairs per key group
  float* bias;      // [NGMAX][GQ] sum_c q_c z_c - sum_c (q*s)_c * offset_c
  float* p;         // [GQ][ST]    logits, then probabilities
  float* red;       // [kRedFloats] value-partial reduction
  float* scratch;   // [64]
};

template <int D, int GQ>
__device__ __forceinline__ Lds carve(unsigned char* smem, int ST, int G) {
  const int ngmax = (ST + G - 1) / G + 1;
  Lds L;
  unsigned char* ptr = smem;
  L.qf = reinterpret_cast<float*>(ptr);       ptr += GQ * D * 4;
  L.qh = reinterpret_cast<uint32_t*>(ptr);    ptr += GQ * D * 2;
  L.qs = reinterpret_cast<uint32_t*>(ptr);    ptr += size_t(ngmax) * GQ * D * 2;
  L.bias = reinterpret_cast<float*>(ptr);     ptr += size_t(ngmax) * GQ * 4;
  L.p = reinterpret_cast<float*>(ptr);        ptr += size_t(GQ) * ST * 4;
  L.red = reinterpret_cast<float*>(ptr);      ptr += size_t(kRedFloats) * 4;
  L.scratch = reinterpret_cast<float*>(ptr);
  return L;
}

// ---------------------------------------------------------------------------
// Keys from a quantized run (bits 2/4/8), tokens [t0, t1) of the split.
template <int D, int GQ, int BITS>
__device__ void keys_quantized(const DecodeParams& P, const Lds& L, int64_t stream,
                               const Run& run, int t0, int t1) {
  constexpr int RB = D * BITS / 8;       // bytes per token row
  constexpr int CPR = RB / 16;           // 16-byte chunks per row
  constexpr int PPC = 64 / BITS;         // fp16 pairs per chunk
  constexpr int NP = Unpack<BITS>::NP;   // pairs per 32-bit word
  constexpr int CPW = 32 / BITS;         // channels per 32-bit word
  constexpr int HD = D / 2;              // pairs per row
  const int ST = P.split_tokens;
  const int G = P.G;
  const int tid = threadIdx.x;
  const int r0 = t0 - run.tok_begin, r1 = t1 - run.tok_begin;
  const int j0 = r0 / G;
  const int ng = (r1 - 1) / G - j0 + 1;
  const uint8_t* codes = P.k_codes + stream * P.k_codes_stride + run.code_off;
  const uint32_t* meta = reinterpret_cast<const uint32_t*>(
      P.k_meta + stream * P.k_meta_stride + run.meta_off);

  // 1. q*s pairs and bias of every group the split touches.  Pair pi of a
  //    row is word w = pi/NP, position k = pi%NP: channels (w*CPW + k) and
  //    (w*CPW + k + NP), the two codes one unpacked word pair holds.
  const int nm = ng * HD;
  for (int base = 0; base < nm; base += NT) {
    const int item = base + tid;
    const bool valid = item < nm;
    const int jl = valid ? item / HD : 0;
    const int pi = item % HD;
    const int w = pi / NP, k = pi % NP;
    const int clo = w * CPW + k, chi = clo + NP;
    uint32_t mlo = 0, mhi = 0;
    if (valid) {
      const uint32_t* m = meta + int64_t(j0 + jl) * D;
      mlo = m[clo];
      mhi = m[chi];
    }
    const float slo = h2f(mlo & 0xffffu), zlo = h2f(mlo >> 16);
    const float shi = h2f(mhi & 0xffffu), zhi = h2f(mhi >> 16);
    const float off = Unpack<BITS>::offset(k);
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      const float qlo = L.qf[h * D + clo], qhi = L.qf[h * D + chi];
      const uint32_t a = f2h(qlo * slo), c = f2h(qhi * shi);
      float bp = qlo * zlo + qhi * zhi - (h2f(a) + h2f(c)) * off;
#pragma unroll
      for (int m = HD / 2; m >= 1; m >>= 1) bp += __shfl_xor(bp, m);
      if (valid) {
        L.qs[(jl * GQ + h) * HD + pi] = a | (c << 16);
        if (pi == 0) L.bias[jl * GQ + h] = bp;
      }
    }
  }
  __syncthreads();

  // 2. logits: item = (token, 16-byte chunk of its row).
  const int ni = (r1 - r0) * CPR;
  for (int base = 0; base < ni; base += NT * U) {
    uint4 cw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int item = base + u * NT + tid;
      if (item < ni) {
        const int r = r0 + item / CPR, c = item % CPR;
        cw[u] = *reinterpret_cast<const uint4*>(codes + int64_t(r) * RB + c * 16);
      } else {
        cw[u] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int item = base + u * NT + tid;
      const bool valid = item < ni;
      const int tl = valid ? item / CPR : 0;
      const int c = item % CPR;
      const int r = r0 + tl;
      const int jl = r / G - j0;
      uint32_t v[4][NP];
      Unpack<BITS>::run(cw[u].x, v[0]);
      Unpack<BITS>::run(cw[u].y, v[1]);
      Unpack<BITS>::run(cw[u].z, v[2]);
      Unpack<BITS>::run(cw[u].w, v[3]);
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        const uint32_t* qs = L.qs + (jl * GQ + h) * HD + c * PPC;
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w)
#pragma unroll
          for (int k = 0; k < NP; ++k) acc = dot2(qs[w * NP + k], v[w][k], acc);
#pragma unroll
        for (int m = CPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
        if (valid && c == 0) L.p[h * ST + (r + run.tok_begin - t0)] = acc + L.bias[jl * GQ + h];
      }
    }
  }
}

// Keys from fp16 rows (the residual, or a 16-bit run): rows[row0 + i], i < nt.
template <int D, int GQ>
__device__ void keys_fp16(const DecodeParams& P, const Lds& L, const uint16_t* rows,
                          int row0, int nt) {
  constexpr int CPR = D / 8;             // 16-byte chunks per row
  const int ST = P.split_tokens;
  const int tid = threadIdx.x;
  const int ni = nt * CPR;
  for (int base = 0; base < ni; base += NT * U) {
    uint4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int item = base + u * NT + tid;
      if (item < ni) {
        x[u] = *reinterpret_cast<const uint4*>(rows + int64_t(row0 + item / CPR) * D + (item % CPR) * 8);
      } else {
        x[u] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int item = base + u * NT + tid;
      const bool valid = item < ni;
      const int tl = valid ? item / CPR : 0;
      const int c = item % CPR;
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        const uint32_t* qh = L.qh + h * (D / 2) + c * 4;
        float acc = dot2(qh[0], x[u].x, 0.f);
        acc = dot2(qh[1], x[u].y, acc);
        acc = dot2(qh[2], x[u].z, acc);
        acc = dot2(qh[3], x[u].w, acc);
#pragma unroll
        for (int m = CPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
        if (valid && c == 0) L.p[h * ST + tl] = acc * P.scale_log2;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Sum the value partials of all threads (slot = threads sharing a channel
// range) and write o[h][:] of this split.
template <int D, int CH>
__device__ __forceinline__ void reduce_write(const Lds& L, const float* vals, int slot,
                                             int ch0, int nslot, float* o) {
  __syncthreads();
#pragma unroll
  for (int j = 0; j < CH; ++j) L.red[slot * D + ch0 + j] = vals[j];
  __syncthreads();
  for (int ch = threadIdx.x; ch < D; ch += NT) {
    float s = 0.f;
    for (int sl = 0; sl < nslot; ++sl) s += L.red[sl * D + ch];
    o[ch] = s;
  }
}

// Values from a quantized run (bits 2/4/8), tokens [t0, t1) of the split.
template <int D, int GQ, int BITS>
__device__ void values_quantized(const DecodeParams& P, const Lds& L, int64_t stream,
                                 const Run& run, int t0, int t1, float* ws) {
  constexpr int RB = D * BITS / 8;
  constexpr int CPP = 2 * RB / 16;        // 16-byte chunks per pair block
  constexpr int CPCV = 64 / BITS;         // channels per chunk
  constexpr int NP = Unpack<BITS>::NP;    // channels per 16-bit unit
  constexpr int HPP = (GQ * CPCV <= 64) ? GQ : ((64 / CPCV) > 0 ? (64 / CPCV) : 1);
  const int ST = P.split_tokens;
  const int G = P.G;
  const int NG = D / G;
  const int tid = threadIdx.x;
  const int c = tid % CPP;                // fixed chunk of this thread
  const int slot = tid / CPP;
  const int g = (c * CPCV) / G;
  const int r0 = t0 - run.tok_begin, r1 = t1 - run.tok_begin;
  const int p0 = r0 >> 1;
  const int np = ((r1 - 1) >> 1) - p0 + 1;
  const int ni = np * CPP;
  const uint8_t* codes = P.v_codes + stream * P.v_codes_stride + run.code_off;
  const uint8_t* meta = P.v_meta + stream * P.v_meta_stride + run.meta_off;

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
    for (int base = 0; base < ni; base += NT * U) {
      uint4 cw[U];
      uint2 mw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int item = base + u * NT + tid;
        if (item < ni) {
          const int64_t pr = p0 + item / CPP;
          cw[u] = *reinterpret_cast<const uint4*>(codes + pr * (2 * RB) + c * 16);
          mw[u] = *reinterpret_cast<const uint2*>(meta + (pr * NG + g) * 8);
        } else {
          cw[u] = make_uint4(0u, 0u, 0u, 0u);
          mw[u] = make_uint2(0u, 0u);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int item = base + u * NT + tid;
        const bool valid = item < ni;
        const int te0 = 2 * (p0 + item / CPP), te1 = te0 + 1;
        const bool ok0 = valid && te0 >= r0 && te0 < r1;
        const bool ok1 = valid && te1 >= r0 && te1 < r1;
        const float s0 = ok0 ? h2f(mw[u].x & 0xffffu) : 0.f, z0 = ok0 ? h2f(mw[u].x >> 16) : 0.f;
        const float s1 = ok1 ? h2f(mw[u].y & 0xffffu) : 0.f, z1 = ok1 ? h2f(mw[u].y >> 16) : 0.f;
        uint32_t v[4][NP];
        Unpack<BITS>::run(cw[u].x, v[0]);
        Unpack<BITS>::run(cw[u].y, v[1]);
        Unpack<BITS>::run(cw[u].z, v[2]);
        Unpack<BITS>::run(cw[u].w, v[3]);
#pragma unroll
        for (int hh = 0; hh < HPP; ++hh) {
          const int h = hp + hh;
          const float pa = ok0 ? L.p[h * ST + te0 - r0] : 0.f;
          const float pb = ok1 ? L.p[h * ST + te1 - r0] : 0.f;
          const uint32_t a = f2h(pa * s0), b = f2h(pb * s1);
          const uint32_t ps = a | (b << 16);
          sps[hh] += h2f(a) + h2f(b);
          pz[hh] += pa * z0 + pb * z1;
#pragma unroll
          for (int w = 0; w < 4; ++w)
#pragma unroll
            for (int k = 0; k < NP; ++k) acc[hh][w * NP + k] = dot2(ps, v[w][k], acc[hh][w * NP + k]);
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < HPP; ++hh) {
      const int h = hp + hh;
      float vals[CPCV];
#pragma unroll
      for (int j = 0; j < CPCV; ++j)
        vals[j] = acc[hh][j] - Unpack<BITS>::offset(j % NP) * sps[hh] + pz[hh];
      float* o = ws + int64_t(h) * (D + 2) + 2;
      if (h < P.gq) reduce_write<D, CPCV>(L, vals, slot, c * CPCV, NT / CPP, o);
    }
  }
}

// Values from fp16 rows: rows[row0 + i], i < nt.
template <int D, int GQ>
__device__ void values_fp16(const DecodeParams& P, const Lds& L, const uint16_t* rows,
                            int row0, int nt, float* ws) {
  constexpr int CPR = D / 8;
  const int ST = P.split_tokens;
  const int tid = threadIdx.x;
  const int c = tid % CPR;
  const int slot = tid / CPR;
  const int ni = nt * CPR;
  float acc[GQ][8];
#pragma unroll
  for (int h = 0; h < GQ; ++h)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[h][j] = 0.f;
  for (int base = 0; base < ni; base += NT * U) {
    uint4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int item = base + u * NT + tid;
      if (item < ni) {
        x[u] = *reinterpret_cast<const uint4*>(rows + int64_t(row0 + item / CPR) * D + c * 8);
      } else {
        x[u] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int item = base + u * NT + tid;
      if (item >= ni) continue;
      const int tl = item / CPR;
      const uint32_t wv[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
      float f[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[2 * e] = h2f(wv[e] & 0xffffu);
        f[2 * e + 1] = h2f(wv[e] >> 16);
      }
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        const float p = L.p[h * ST + tl];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] += p * f[j];
      }
    }
  }
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    float* o = ws + int64_t(h) * (D + 2) + 2;
    if (h < P.gq) reduce_write<D, 8>(L, acc[h], slot, c * 8, NT / CPR, o);
  }
}

// ---------------------------------------------------------------------------
template <int D, int GQ>
__global__ void __launch_bounds__(NT) decode_split_kernel(const DecodeParams P) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int ST = P.split_tokens;
  const Lds L = carve<D, GQ>(smem, ST, P.G);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x;
  const int64_t stream = blockIdx.y;
  const int b = int(stream / P.Hkv), hkv = int(stream % P.Hkv);

  int ci = 0;
  while (ci + 1 < P.n_cells && P.cells[ci + 1].split0 <= split) ++ci;
  const Cell cell = P.cells[ci];
  const int t0 = cell.t0 + (split - cell.split0) * ST;
  const int t1 = min(t0 + ST, cell.t0 + cell.n);
  const int nt = t1 - t0;

  const int64_t qrow = (int64_t(b) * P.Hq + int64_t(hkv) * P.gq) * D;
  for (int i = tid; i < GQ * D; i += NT) {
    const int h = i / D, ch = i % D;
    L.qf[i] = h < P.gq ? h2f(P.q[qrow + int64_t(h) * D + ch]) * P.scale_log2 : 0.f;
  }
  const uint32_t* q32 = reinterpret_cast<const uint32_t*>(P.q);
  for (int i = tid; i < GQ * (D / 2); i += NT) {
    const int h = i / (D / 2), c2 = i % (D / 2);
    L.qh[i] = h < P.gq ? q32[(qrow + int64_t(h) * D) / 2 + c2] : 0u;
  }
  __syncthreads();

  if (cell.k_src >= 0) {
    const Run& run = P.k_runs[cell.k_src];
    switch (run.bits) {
      case 2: keys_quantized<D, GQ, 2>(P, L, stream, run, t0, t1); break;
      case 4: keys_quantized<D, GQ, 4>(P, L, stream, run, t0, t1); break;
      case 8: keys_quantized<D, GQ, 8>(P, L, stream, run, t0, t1); break;
      default:
        keys_fp16<D, GQ>(P, L,
                         reinterpret_cast<const uint16_t*>(P.k_codes + stream * P.k_codes_stride + run.code_off),
                         t0 - run.tok_begin, nt);
    }
  } else {
    keys_fp16<D, GQ>(P, L, P.k_res + stream * P.k_res_stride, t0 - P.n_kq, nt);
  }
  __syncthreads();

  // split-local softmax state per head (base-2 logits)
  float mh[GQ], lh[GQ];
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    float mx = -INFINITY;
    for (int i = tid; i < nt; i += NT) mx = fmaxf(mx, L.p[h * ST + i]);
    mx = wave_max(mx);
    if (lane == 0) L.scratch[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(L.scratch[0], L.scratch[1]), fmaxf(L.scratch[2], L.scratch[3]));
    __syncthreads();
    float sum = 0.f;
    for (int i = tid; i < nt; i += NT) {
      const float e = exp2f(L.p[h * ST + i] - mx);
      L.p[h * ST + i] = e;
      sum += e;
    }
    sum = wave_sum(sum);
    if (lane == 0) L.scratch[wave] = sum;
    __syncthreads();
    sum = L.scratch[0] + L.scratch[1] + L.scratch[2] + L.scratch[3];
    __syncthreads();
    mh[h] = mx;
    lh[h] = sum;
  }

  float* ws = P.ws + (stream * P.n_splits + split) * int64_t(P.gq) * (D + 2);
  if (cell.v_src >= 0) {
    const Run& run = P.v_runs[cell.v_src];
    switch (run.bits) {
      case 2: values_quantized<D, GQ, 2>(P, L, stream, run, t0, t1, ws); break;
      case 4: values_quantized<D, GQ, 4>(P, L, stream, run, t0, t1, ws); break;
      case 8: values_quantized<D, GQ, 8>(P, L, stream, run, t0, t1, ws); break;
      default:
        values_fp16<D, GQ>(P, L,
                           reinterpret_cast<const uint16_t*>(P.v_codes + stream * P.v_codes_stride + run.code_off),
                           t0 - run.tok_begin, nt, ws);
    }
  } else {
    values_fp16<D, GQ>(P, L, P.v_res + stream * P.v_res_stride, t0 - P.n_vq, nt, ws);
  }
  if (tid == 0) {
    for (int h = 0; h < GQ && h < P.gq; ++h) {
      ws[int64_t(h) * (D + 2)] = mh[h];
      ws[int64_t(h) * (D + 2) + 1] = lh[h];
    }
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
  const size_t lds = size_t(decode_lds_bytes(D, GQ, p.split_tokens, p.G));
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
