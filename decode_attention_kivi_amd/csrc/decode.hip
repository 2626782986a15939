// Decode-step attention over a low-bit quantized KV cache, split over the
// context (the FlashDecoding dataflow that the VQ-LLM note's reference [10]
// describes) with a cross-split softmax merge.
//
// The N tokens of a cache stream (batch b, kv head h) are cut into
// waves_per_stream ranges of about equal HBM bytes (starts at multiples of 32);
// a workgroup holds eight consecutive ranges of one stream and the GQ query
// heads that share it.  A wave's range may cross run boundaries: it walks the
// key pieces (quantized runs, fp16 runs, the fp16 residual) and then the value
// pieces in token order.  Per wave:
//   1. logits, one load batch at a time: quarter-row code loads, the batch's
//      key groups' q*s (per-channel key scales, KIVI note "Method details") as
//      fp16 hi + lo rows of a matrix-core A operand and the group biases
//      sum_c q_c z_c into LDS; code pairs are unpacked into fp16 (offset +
//      code) by mask-and-or with an exponent constant and form the B operand
//      of v_mfma_f32_16x16x32_f16 (16 tokens per instruction group); residual
//      rows dot q directly (A = Concat([A_g, A_r]));
//   2. the range's max and sum of exp2(logit - max): one softmax over the
//      concatenation (KIVI Algorithm 1; WindowQuant Sec. 3.3.1);
//   3. A.V over token-pair value blocks: one fp16 pair holds the same channel
//      of two tokens, so v_dot2 applies both tokens' p*s at once; sum(p*s) and
//      sum(p*z) of a lane are kept apart and folded in after the cross-lane
//      reduction;
//   4. the eight waves' (max, sum, o[d]) are combined: into the output when
//      one workgroup covers the stream, otherwise into the workgroup's
//      partial state, which a second kernel merges with the stream's others.
// Logits stay raw q'.k (q' = q * 2^-8, exact) until the softmax scales them
// by sm_scale * log2(e) * 2^8 into base-2 logits.

#include "kvq_internal.h"
#include "kvq_device.h"
#include "kvq_quant.h"

namespace kvq {
namespace {

// Waves per SIMD of the decode kernel: four for one query head per kv head,
// three for head blocks of 4 at d_h = 128 (168 VGPRs), two otherwise.
constexpr int decode_waves_per_simd(int D, int GQ) { return GQ == 1 ? 4 : decode_waves(D, GQ) == 12 ? 3 : 2; }
// Load batches in flight per wave in the streaming loops: three at two waves
// per SIMD (registers to spare), two otherwise.
template <int D, int GQ> constexpr int stream_batches() { return decode_waves_per_simd(D, GQ) == 2 ? 3 : 2; }
// Loads per batch in the value pair loop (two batches in flight): grouped
// heads at two waves per SIMD keep more loads in flight per wave.
template <int GQ> constexpr int value_batch() { return GQ == 1 ? 2 : 3; }

// Make this wave's LDS writes visible to its own later LDS reads.  LDS
// operations of one wave execute in order; this only keeps the compiler from
// moving memory operations across the point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half2_t as_h2(uint32_t x) { return __builtin_bit_cast(half2_t, x); }
__device__ __forceinline__ uint32_t as_u32(half2_t x) { return __builtin_bit_cast(uint32_t, x); }

// Issue priority from the wave's progress through its range (keys, then
// values; four levels, a wave that is behind gets a higher one).  The waves
// of two workgroups share each CU; the issue arbiter otherwise favours the
// older workgroup, which then finishes far earlier and leaves the younger one
// to run the tail at half occupancy.
__device__ __forceinline__ void progress_prio(int phase, int done, int total) {
  const int level = 3 - 2 * phase - (2 * done >= total ? 1 : 0);
  switch (level) {
    case 3: __builtin_amdgcn_s_setprio(3); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    default: __builtin_amdgcn_s_setprio(0); break;
  }
}

template <int W> struct LoadType;
template <> struct LoadType<1> { typedef uint32_t T; };
template <> struct LoadType<2> { typedef uint2 T; };
template <> struct LoadType<4> { typedef uint4 T; };
struct Words8 { uint4 a, b; };
template <> struct LoadType<8> { typedef Words8 T; };

template <int W>
__device__ __forceinline__ uint32_t word(const typename LoadType<W>::T& x, int i) {
  if constexpr (W == 1) {
    return x;
  } else if constexpr (W == 2) {
    return i == 0 ? x.x : x.y;
  } else if constexpr (W == 4) {
    return i == 0 ? x.x : i == 1 ? x.y : i == 2 ? x.z : x.w;
  } else {
    const uint4& y = i < 4 ? x.a : x.b;
    const int k = i & 3;
    return k == 0 ? y.x : k == 1 ? y.y : k == 2 ? y.z : y.w;
  }
}

// Range-checked loads: a raw buffer resource over [base, base + bytes);
// reads at or past the end return zeros (no clamping, no fault).  Offsets
// stay in the per-lane register and the instruction's immediate.
//
// Every byte of the cache is read once per call, so the loads carry the
// non-temporal cache policy (nt): a plain streaming read of the decode
// launch's bytes ran 11% faster with it on MI355X (31.9 us against 35.8 us
// for 215 MB), and the traffic counters show no extra HBM reads.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kStreamAux = 2;   // cache policy bits of the streaming loads: nt
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), short(0), int(bytes), 0x00020000);
}
template <int W>
__device__ __forceinline__ typename LoadType<W>::T bload(Rsrc r, uint32_t off) {
  if constexpr (W == 1) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kStreamAux);
  } else if constexpr (W == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kStreamAux);
    return make_uint2(v[0], v[1]);
  } else if constexpr (W == 4) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStreamAux);
    return make_uint4(v[0], v[1], v[2], v[3]);
  } else {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStreamAux);
    const auto w = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, kStreamAux);
    return Words8{make_uint4(v[0], v[1], v[2], v[3]), make_uint4(w[0], w[1], w[2], w[3])};
  }
}

struct WaveLds {
  float* logit;      // [GQ][LT] logits by token slot
  uint16_t* p16;     // [GQ][LT] fp16 probabilities, zero outside the wave's tokens
  float* red;        // the value reduction's row sums (after the softmax)
  uint32_t* qs;      // [NGB][QBLK] A blocks (q*s hi/lo rows) of one load batch
  float* bias;       // [NGB][GQ] key biases per (group, head), after the largest A blocks
  float* ow;         // [GQ][D+2] (m, l, o[D]) of the wave (aliases qs/bias)
};

template <int D, int GQ>
__device__ __forceinline__ WaveLds carve_wave(unsigned char* smem, int wave) {
  constexpr DecodeLds lay = decode_lds<D, GQ>();
  constexpr int64_t QSMAX = kQsMax<D, GQ>();
  unsigned char* base = smem + lay.block + int64_t(wave) * lay.wave;
  WaveLds W;
  W.logit = reinterpret_cast<float*>(base);
  if constexpr (p16_over_logits(GQ)) {
    W.p16 = reinterpret_cast<uint16_t*>(base);
    W.red = W.logit + GQ * wave_slots(GQ) / 2;
  } else {
    W.p16 = reinterpret_cast<uint16_t*>(base + lay.logit);
    W.red = W.logit;
  }
  W.qs = reinterpret_cast<uint32_t*>(base + lay.logit + lay.p16);
  W.bias = reinterpret_cast<float*>(W.qs + QSMAX);
  W.ow = reinterpret_cast<float*>(base + lay.logit + lay.p16);
  return W;
}

// ---------------------------------------------------------------------------
// Page cursor of a paged cache: the buffers that hold a sequence's key (or
// value) tokens, page by page, for loops that run one load pipeline across
// page boundaries.  Tokens are sequence tokens; code and meta units are
// tokens or pairs (codes) and key groups or pairs (meta), 2^lg_cu and 2^lg_mu
// tokens each.  Lane i holds the pool page of the sequence's page pg0 + i
// (a wave's range spans far fewer than 64 pages); at(t) moves the cursor
// forward to the page of token t (calls come in token order) and keeps buffer
// resources for that page and the next, so that a load batch (at most
// 64 tokens, a page at least 64) finds every token in one of the two.
// Tokens of a page past the run's n_valid tokens read as zeros.
struct PageLoc {
  const uint8_t* head;                // pool base + kv head block offset
  int64_t page_bytes;
  int32_t PT, c_off, m_off, n_valid;
  int32_t lg_cu, cu_bytes, lg_mu, mu_bytes;
  int32_t pg0, my_page;
  int32_t pa, end_a;                  // current page, its end token
  Rsrc ca, cb, ma, mb;                // codes / meta of page pa and pa + 1
  __device__ __forceinline__ void start(const int32_t* row, int32_t max_pages, int t0, int lane) {
    pg0 = t0 / PT;
    my_page = row[min(pg0 + lane, max_pages - 1)];
    pa = pg0;
    end_a = (pg0 + 1) * PT;
    load(pa);
  }
  __device__ __forceinline__ Rsrc page(int pg, int32_t off, int lg, int unit) const {
    const int k = pg - pg0;
    const int v = k < 64 ? min(max(n_valid - pg * PT, 0), PT) : 0;   // valid tokens of the page
    const int32_t id = __builtin_amdgcn_readlane(my_page, min(k, 63));
    return make_rsrc(head + int64_t(id) * page_bytes + off, uint32_t(((v + (1 << lg) - 1) >> lg) * unit));
  }
  __device__ __forceinline__ void load(int pg) {
    ca = page(pg, c_off, lg_cu, cu_bytes);
    cb = page(pg + 1, c_off, lg_cu, cu_bytes);
    ma = page(pg, m_off, lg_mu, mu_bytes);
    mb = page(pg + 1, m_off, lg_mu, mu_bytes);
  }
  __device__ __forceinline__ void at(int t) {
    if (t >= end_a) {                 // (uniform)
      do {
        ++pa;
        end_a += PT;
      } while (t >= end_a);
      load(pa);
    }
  }
  // buffer and byte offset of token t's code unit / meta unit (t in page pa or pa + 1)
  __device__ __forceinline__ Rsrc code(int t, uint32_t& off) const {
    const bool nx = t >= end_a;
    off = uint32_t(((t - (nx ? end_a : end_a - PT)) >> lg_cu) * cu_bytes);
    return nx ? cb : ca;
  }
  __device__ __forceinline__ Rsrc meta(int t, uint32_t& off) const {
    const bool nx = t >= end_a;
    off = uint32_t(((t - (nx ? end_a : end_a - PT)) >> lg_mu) * mu_bytes);
    return nx ? mb : ma;
  }
};

// ---------------------------------------------------------------------------
// Keys of run tokens [r0, r1) (bits 2/4/8) -> raw logits q'.k (q' = q * 2^-8)
// at slots slot0 + (t - r0); cbase / mbase address the run's token 0 (codes)
// and key group 0 (meta) of this stream.  r0 is a multiple of 32, so every
// item (16 tokens) lies in one key group.  Whole items are written: slots past r1 get
// values that a later piece overwrites or the softmax ignores.
//
// Per key group, every channel's hi = fp16(q'*s) and lo = fp16(q'*s - hi)
// (packed fp16 ops; q' = q * 2^-8 exactly): a single fp16 q*s is too coarse
// for outlier channels, whose large logits would carry its 2^-11 relative
// error into the softmax.  hi and lo of head h are rows 2h and 2h+1 of the A
// operand of v_mfma_f32_16x16x32_f16; B is the unpacked codes of 16 tokens,
// (offset + code) per channel, so D[2h][t] + D[2h+1][t] plus the group's bias
// sum_c q'_c z_c - sum_c (hi + lo)_c * offset_c is the logit of token t (the
// bias is reduced over the row's channels once per group).
//
// Operand layout (16x16x32): lane l holds A[l % 16][8*(l/16) .. +8),
// B[8*(l/16) .. +8][l % 16] and D[4*(l/16) .. +4][l % 16].  k-block l/16 of
// instruction m is code pairs 4m .. 4m+3 of the lane's quarter row (pair P:
// word P / NP, position P % NP, channels clo and clo + NP).
template <int D, int GQ, int BITS, bool PG = false>
__device__ __forceinline__ void keys_quantized(const DecodeParams& P, const WaveLds& W, const uint16_t* qg, int nh,
                               const uint8_t* cbase, const uint8_t* mbase, int r0, int r1, int slot0,
                               int lane, int n_wave, PageLoc* loc = nullptr) {
  using KG = KeyGeo<D, GQ, BITS>;
  constexpr int LT = wave_slots(GQ);
  constexpr int RB = KG::RB, LB = KG::LB, TPI = KG::TPI, WPL = KG::WPL, MF = KG::MF;
  constexpr int NP = KG::NP, CPW = KG::CPW, PPL = KG::PPL, HD = KG::HD;
  constexpr int NB = KG::NB, NGB = KG::NGB, ROWS = KG::ROWS, BS = KG::BS, QBLK = KG::QBLK;
  constexpr int GPI = 64 / HD;                         // key groups per meta iteration
  constexpr int MI = (NGB + GPI - 1) / GPI;
  const int lg = P.lg_g;
  const int n = r1 - r0;
  const int n_items = (n + TPI - 1) / TPI;
  const int jp = r0 >> lg;                             // first key group of the piece
  const int n_groups = ((r1 - 1) >> lg) - jp + 1;
  // (paged: the page cursor supplies the buffers; cbase and mbase are null)
  const Rsrc crs = make_rsrc(cbase + (PG ? 0 : int64_t(r0) * RB), PG ? 0u : uint32_t(n) * RB);
  const Rsrc mrs = make_rsrc(mbase + (PG ? 0 : int64_t(jp) * D * 4), PG ? 0u : uint32_t(n_groups) * D * 4);
  // matrix role of the lane: B column (token) col, k-block kb; A row col
  const int col = lane & 15, kb = lane >> 4;
  const uint32_t lane_off = uint32_t(col * RB + kb * LB);
  // LDS dword of the lane's A row in block (m = 0, kb) of a group.  Rows past
  // 2*GQ repeat row col % (2*GQ): they only feed D rows that are never read.
  const int a_pos = kb * BS + (col & (ROWS - 1)) * 4;
  // the lane's logit slots (token col of each item) for heads 2kb and 2kb + 1
  float* const lgs = W.logit + (2 * kb) * LT + slot0 + col;

  // meta role of the lane: pair pi of a row of group gsub (of the meta
  // iteration): k-block pj, pair pp of it
  const int pi = lane % HD, gsub = lane / HD;
  const int pj = pi / PPL, pp = pi % PPL;
  const int kq = pp % NP;
  const int clo = pj * (D / 4) + (pp / NP) * CPW + kq, chi = clo + NP;
  const int qpos = ((pp / 4) * 4 + pj) * BS + pp % 4;   // its hi dword in block [pp/4][pj]
  const uint32_t meta_off = uint32_t((gsub * D + clo) * 4);
  const Unpacker<BITS, false> unpack;                 // constants in registers, once
  const _Float16 off = static_cast<_Float16>(Unpacker<BITS, false>::offset(kq));
  const half2_t nego = {-off, -off};

  half2_t qk[GQ];

  // Software pipeline over load batches: the loads of batch b+1 are in
  // flight while batch b is consumed.  A batch past the end is still issued:
  // its reads fall outside the buffer ranges and return zeros without
  // touching memory, and issuing unconditionally keeps the wait counts exact.
  struct Batch {
    typename LoadType<WPL>::T buf[NB];
    uint32_t mlo[MI], mhi[MI];
  };
  auto issue = [&](Batch& B, int i0) {
    if constexpr (PG) {
      // pages: each item and each group lies in one page (pages hold whole
      // groups and multiples of 64 tokens)
      static_assert(GPI == 1, "one key group per meta iteration");
      const int t = r0 + i0 * TPI;
      loc->at(t);
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        uint32_t o;
        const Rsrc rs = loc->code(t + u * TPI, o);
        B.buf[u] = bload<WPL>(rs, o + lane_off);
      }
#pragma unroll
      for (int it = 0; it < MI; ++it) {
        uint32_t o;
        const Rsrc rs = loc->meta(((t >> lg) + it) << lg, o);
        B.mlo[it] = bload<1>(rs, o + meta_off);
        B.mhi[it] = bload<1>(rs, o + meta_off + NP * 4);
      }
    } else {
      const uint32_t cb = lane_off + uint32_t(i0 * TPI * RB);
#pragma unroll
      for (int u = 0; u < NB; ++u) B.buf[u] = bload<WPL>(crs, cb + u * TPI * RB);
      const uint32_t mb = meta_off + uint32_t((((r0 + i0 * TPI) >> lg) - jp) * D * 4);
#pragma unroll
      for (int it = 0; it < MI; ++it) {
        B.mlo[it] = bload<1>(mrs, mb + it * GPI * D * 4);
        B.mhi[it] = bload<1>(mrs, mb + it * GPI * D * 4 + NP * 4);
      }
    }
  };
  auto consume = [&](const Batch& B, int i0) {
    const int jb0 = ((r0 + i0 * TPI) >> lg) - jp;      // batch groups, relative to the piece
    const int ng = min(((r0 + min((i0 + NB) * TPI, n) - 1) >> lg) - jp - jb0 + 1, NGB);
    float bpv[MI][GQ];                       // the lane's bias terms
#pragma unroll
    for (int it = 0; it < MI; ++it) {
#pragma unroll
      for (int h = 0; h < GQ; ++h) bpv[it][h] = 0.f;
      if (it * GPI >= ng) continue;          // uniform; keeps the loop fully unrolled
      const int js = it * GPI + gsub;
      const half2_t s2 = as_h2(__builtin_amdgcn_perm(B.mhi[it], B.mlo[it], 0x05040100u));
      const half2_t z2 = as_h2(__builtin_amdgcn_perm(B.mhi[it], B.mlo[it], 0x07060302u));
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        const half2_t hi = qk[h] * s2;
        const half2_t lo = __builtin_elementwise_fma(qk[h], s2, -hi);
        float bp = __builtin_amdgcn_fdot2(qk[h], z2, 0.f, false);
        bp = __builtin_amdgcn_fdot2(hi, nego, bp, false);
        bpv[it][h] = __builtin_amdgcn_fdot2(lo, nego, bp, false);
        if (js < ng) {
          uint32_t* qs = W.qs + js * QBLK + qpos;
          qs[(2 * h) * 4] = as_u32(hi);
          qs[(2 * h + 1) * 4] = as_u32(lo);
        }
      }
    }
    // biases: sums of the terms over the HD pairs of a row
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      if constexpr (MI == 2 && GPI == 1) {
        // both groups at once: fold the wave halves so that lanes 0-31 hold
        // group 0's terms and lanes 32-63 group 1's, then sum 32 lanes
        const auto r = __builtin_amdgcn_permlane32_swap(fbits(bpv[0][h]), fbits(bpv[1][h]), false, false);
        const float x = xrow_sum<2>(group_sum<16>(bitsf(r[0]) + bitsf(r[1])));
        if ((lane & 31) == 0 && (lane >> 5) < ng) W.bias[(lane >> 5) * GQ + h] = x;
      } else {
#pragma unroll
        for (int it = 0; it < MI; ++it) {
          if (it * GPI >= ng) continue;
          const float x = xrow_sum<HD / 16>(group_sum<16>(bpv[it][h]));
          if (pi == 0 && it * GPI + gsub < ng) W.bias[(it * GPI + gsub) * GQ + h] = x;
        }
      }
    }
    wave_lds_sync();

    half8_t am[MF];
    float b0 = 0.f, b1 = 0.f;
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int i = i0 + u;
      if (i >= n_items) continue;            // uniform
      const int rt = r0 + i * TPI;           // first run token of the item
      if (u == 0 || (rt & (P.G - 1)) == 0) {
        // (uniform) the item starts a group: fetch the lane's A row and the
        // biases of the heads whose rows its D registers hold
        const int js = min((rt >> lg) - jp - jb0, NGB - 1);
        const uint32_t* qs = W.qs + js * QBLK + a_pos;
#pragma unroll
        for (int m = 0; m < MF; ++m)
          am[m] = __builtin_bit_cast(half8_t, *reinterpret_cast<const uint4*>(qs + m * 4 * BS));
        b0 = W.bias[js * GQ + (2 * kb < GQ ? 2 * kb : 0)];
        if (GQ > 1) b1 = W.bias[js * GQ + (2 * kb + 1 < GQ ? 2 * kb + 1 : 0)];
      }
      uint32_t v[PPL];
#pragma unroll
      for (int w = 0; w < WPL; ++w) unpack.run(word<WPL>(B.buf[u], w), v + w * NP);
      float4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < MF; ++m) {
        const uint4 bm = make_uint4(v[4 * m], v[4 * m + 1], v[4 * m + 2], v[4 * m + 3]);
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(am[m], __builtin_bit_cast(half8_t, bm), d, 0, 0, 0);
      }
      // lane (kb, col) holds rows 4kb .. 4kb+3: heads 2kb and 2kb + 1
      if (2 * kb < GQ) lgs[i * TPI] = (d[0] + b0) + d[1];
      if (2 * kb + 1 < GQ) lgs[LT + i * TPI] = (d[2] + b1) + d[3];
    }
    wave_lds_sync();                         // the next batch rewrites the A blocks
  };

  Batch A, Bb, Cc;
  issue(A, 0);
  if constexpr (stream_batches<D, GQ>() == 3) issue(Bb, NB);
  // q of the lane's meta pair for the GQ heads (global, cached), loaded while
  // the first batch is in flight; padded heads are zero
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    const uint32_t q2 = h < nh ? uint32_t(qg[h * D + clo]) | (uint32_t(qg[h * D + chi]) << 16) : 0u;
    qk[h] = as_h2(q2) * as_h2(0x1C001C00u);                       // * 2^-8, exact
  }
  if constexpr (stream_batches<D, GQ>() == 3) {
    for (int i0 = 0; i0 < n_items; i0 += 3 * NB) {
      progress_prio(0, slot0 + i0 * TPI, n_wave);
      issue(Cc, i0 + 2 * NB);
      consume(A, i0);
      issue(A, i0 + 3 * NB);
      if (i0 + NB < n_items) consume(Bb, i0 + NB);
      issue(Bb, i0 + 4 * NB);
      if (i0 + 2 * NB < n_items) consume(Cc, i0 + 2 * NB);
    }
  } else {
    for (int i0 = 0; i0 < n_items; i0 += 2 * NB) {
      progress_prio(0, slot0 + i0 * TPI, n_wave);
      issue(Bb, i0 + NB);
      consume(A, i0);
      issue(A, i0 + 2 * NB);
      if (i0 + NB < n_items) consume(Bb, i0 + NB);
    }
  }
}

// The key loop on v_dot2 instead of matrix cores, for one query head per kv
// head.  It is compiled only into the comparison library that the build
// makes on request (KVQ_KEY_LOOP_DOT2 defined), to measure the matrix-core
// loop against: the same code loads, meta loads and unpacking; per key group
// hi = fp16(q'*s) and lo = fp16(q'*s - hi) of every channel pair go to LDS
// in lane-chunk order, and per item each lane applies them to its unpacked
// pairs with two v_dot2 per pair, its accumulator seeded with the chunk's
// share of the bias sum_c q'_c z_c - sum_c (hi + lo)_c offset_c; a DPP sum
// over the lanes of a token row gives the logit.
#ifdef KVQ_KEY_LOOP_DOT2
constexpr bool kKeyLoopDot2 = true;
#else
constexpr bool kKeyLoopDot2 = false;
#endif

template <int D, int BITS>
struct KeyGeoDot2 {
  static constexpr int RB = D * BITS / 8;       // bytes per token row
  static constexpr int NP = 16 / BITS;          // fp16 code pairs per 32-bit word
  static constexpr int CPW = 32 / BITS;         // channels per 32-bit word
  static constexpr int LB0 = 4 * 16 / NP;
  static constexpr int LB = LB0 > 16 ? (RB < 16 ? RB : 16) : (LB0 > RB ? RB : LB0);
  static constexpr int LPR = RB / LB;           // lanes per token row
  static constexpr int TPI = 64 / LPR;          // tokens per wave instruction (item)
  static constexpr int WPL = LB / 4;            // code words per lane
  static constexpr int PPL = WPL * NP;          // code pairs per lane
  static constexpr int HD = D / 2;              // code pairs per row
  static constexpr int NB = 4;                  // items per load batch
  static constexpr int NGB = NB * TPI / 32 > 1 ? NB * TPI / 32 : 1;  // key groups per batch
  static constexpr int QSTR = PPL + 4;          // LDS dwords per lane chunk (padded)
  static constexpr int QGRP = 2 * LPR * QSTR;   // LDS dwords per group: hi chunks, then lo chunks
  static_assert(LPR * PPL == HD, "lanes of a row cover its pairs");
  static_assert(TPI <= 32 && (NB * TPI) % 32 == 0, "items never straddle a key group");
  static_assert(NGB * (QGRP + LPR) <= kQsMax<D, 1>() + kBiasMax<D, 1>(), "fits the A-block area");
};

template <int D, int BITS>
__device__ __forceinline__ void keys_quantized_dot2(const DecodeParams& P, const WaveLds& W, const uint16_t* qg,
                                                    int nh, const uint8_t* cbase, const uint8_t* mbase, int r0,
                                                    int r1, int slot0, int lane, int n_wave) {
  using KG = KeyGeoDot2<D, BITS>;
  constexpr int LT = wave_slots(1);
  constexpr int RB = KG::RB, LB = KG::LB, LPR = KG::LPR, TPI = KG::TPI, WPL = KG::WPL;
  constexpr int NP = KG::NP, CPW = KG::CPW, PPL = KG::PPL, HD = KG::HD;
  constexpr int NB = KG::NB, NGB = KG::NGB, QSTR = KG::QSTR, QGRP = KG::QGRP;
  constexpr int GPI = 64 / HD;                         // key groups per meta iteration
  constexpr int MI = (NGB + GPI - 1) / GPI;
  const int lg = P.lg_g;
  const int n = r1 - r0;
  const int n_items = (n + TPI - 1) / TPI;
  const int jp = r0 >> lg;
  const int n_groups = ((r1 - 1) >> lg) - jp + 1;
  const Rsrc crs = make_rsrc(cbase + int64_t(r0) * RB, uint32_t(n) * RB);
  const Rsrc mrs = make_rsrc(mbase + int64_t(jp) * D * 4, uint32_t(n_groups) * D * 4);
  const int tt = lane / LPR, tq = lane % LPR;          // token of the item, chunk of its row
  const uint32_t lane_off = uint32_t(tt * RB + tq * LB);
  uint32_t* qsb = W.qs;                                // [NGB][QGRP] q*s chunks
  float* bsb = reinterpret_cast<float*>(W.qs + NGB * QGRP);   // [NGB][LPR] chunk biases

  // meta role: pair pi of a row (channels clo and clo + NP) of group gsub
  const int pi = lane % HD, gsub = lane / HD;
  const int kq = pi % NP;
  const int clo = (pi / NP) * CPW + kq, chi = clo + NP;
  const int qpos = (pi / PPL) * QSTR + pi % PPL;       // LDS dword of the pair's hi in its chunk
  const uint32_t meta_off = uint32_t((gsub * D + clo) * 4);
  const Unpacker<BITS, false> unpack;
  const _Float16 off = static_cast<_Float16>(Unpacker<BITS, false>::offset(kq));
  const half2_t nego = {-off, -off};
  const uint32_t q2 = nh > 0 ? uint32_t(qg[clo]) | (uint32_t(qg[chi]) << 16) : 0u;
  const half2_t qk = as_h2(q2) * as_h2(0x1C001C00u);   // * 2^-8, exact

  struct Batch {
    typename LoadType<WPL>::T buf[NB];
    uint32_t mlo[MI], mhi[MI];
  };
  auto issue = [&](Batch& B, int i0) {
    const uint32_t cb = lane_off + uint32_t(i0 * TPI * RB);
#pragma unroll
    for (int u = 0; u < NB; ++u) B.buf[u] = bload<WPL>(crs, cb + u * TPI * RB);
    const uint32_t mb = meta_off + uint32_t((((r0 + i0 * TPI) >> lg) - jp) * D * 4);
#pragma unroll
    for (int it = 0; it < MI; ++it) {
      B.mlo[it] = bload<1>(mrs, mb + it * GPI * D * 4);
      B.mhi[it] = bload<1>(mrs, mb + it * GPI * D * 4 + NP * 4);
    }
  };
  auto consume = [&](const Batch& B, int i0) {
    const int jb0 = ((r0 + i0 * TPI) >> lg) - jp;
    const int ng = min(((r0 + min((i0 + NB) * TPI, n) - 1) >> lg) - jp - jb0 + 1, NGB);
#pragma unroll
    for (int it = 0; it < MI; ++it) {
      if (it * GPI >= ng) continue;                    // uniform
      const int js = it * GPI + gsub;
      const half2_t s2 = as_h2(__builtin_amdgcn_perm(B.mhi[it], B.mlo[it], 0x05040100u));
      const half2_t z2 = as_h2(__builtin_amdgcn_perm(B.mhi[it], B.mlo[it], 0x07060302u));
      const half2_t hi = qk * s2;
      const half2_t lo = __builtin_elementwise_fma(qk, s2, -hi);
      float bp = __builtin_amdgcn_fdot2(qk, z2, 0.f, false);
      bp = __builtin_amdgcn_fdot2(hi, nego, bp, false);
      bp = __builtin_amdgcn_fdot2(lo, nego, bp, false);
      bp = group_sum<PPL>(bp);
      if (js < ng) {
        qsb[js * QGRP + qpos] = as_u32(hi);
        qsb[js * QGRP + LPR * QSTR + qpos] = as_u32(lo);
        if (pi % PPL == 0) bsb[js * LPR + pi / PPL] = bp;
      }
    }
    wave_lds_sync();
    uint32_t qhi[PPL], qlo[PPL];
    float bias = 0.f;
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int i = i0 + u;
      if (i >= n_items) continue;                      // uniform
      const int rt = r0 + i * TPI;
      if (u == 0 || (rt & (P.G - 1)) == 0) {
        const int js = min((rt >> lg) - jp - jb0, NGB - 1);
        const uint32_t* qs = qsb + js * QGRP + tq * QSTR;
#pragma unroll
        for (int p = 0; p < PPL; p += 4) {
          const uint4 x = *reinterpret_cast<const uint4*>(qs + p);
          const uint4 y = *reinterpret_cast<const uint4*>(qs + LPR * QSTR + p);
          qhi[p] = x.x; qhi[p + 1] = x.y; qhi[p + 2] = x.z; qhi[p + 3] = x.w;
          qlo[p] = y.x; qlo[p + 1] = y.y; qlo[p + 2] = y.z; qlo[p + 3] = y.w;
        }
        bias = bsb[js * LPR + tq];
      }
      float acc = bias;
#pragma unroll
      for (int w = 0; w < WPL; ++w) {
        uint32_t v[NP];
        unpack.run(word<WPL>(B.buf[u], w), v);
#pragma unroll
        for (int k = 0; k < NP; ++k) {
          acc = dot2(qhi[w * NP + k], v[k], acc);
          acc = dot2(qlo[w * NP + k], v[k], acc);
        }
      }
      W.logit[slot0 + i * TPI + tt] = group_sum<LPR>(acc);
    }
    wave_lds_sync();
  };

  Batch A, Bb;
  issue(A, 0);
  for (int i0 = 0; i0 < n_items; i0 += 2 * NB) {
    progress_prio(0, slot0 + i0 * TPI, n_wave);
    issue(Bb, i0 + NB);
    consume(A, i0);
    issue(A, i0 + 2 * NB);
    if (i0 + NB < n_items) consume(Bb, i0 + NB);
  }
}

// Quantized keys: matrix cores (the comparison library: v_dot2 for one head
// at d_h = 128).
template <int D, int GQ, int BITS, bool PG = false>
__device__ __forceinline__ void keys_q(const DecodeParams& P, const WaveLds& W, const uint16_t* qg, int nh,
                                       const uint8_t* cbase, const uint8_t* mbase, int r0, int r1, int slot0,
                                       int lane, int n_wave, PageLoc* loc = nullptr) {
  if constexpr (PG)
    keys_quantized<D, GQ, BITS, true>(P, W, qg, nh, cbase, mbase, r0, r1, slot0, lane, n_wave, loc);
  else if constexpr (kKeyLoopDot2 && GQ == 1 && D == 128)
    keys_quantized_dot2<D, BITS>(P, W, qg, nh, cbase, mbase, r0, r1, slot0, lane, n_wave);
  else
    keys_quantized<D, GQ, BITS>(P, W, qg, nh, cbase, mbase, r0, r1, slot0, lane, n_wave);
}

// Keys from fp16 rows rows[0..n) -> raw logits q'.k at slots slot0 + i
// (whole items are written, as above).
template <int D, int GQ>
__device__ __forceinline__ void keys_fp16(const DecodeParams& P, const WaveLds& W, const uint16_t* qg, int nh,
                          const uint16_t* rows, int n, int slot0, int lane) {
  constexpr int LT = wave_slots(GQ);
  constexpr int CPR = D / 8;             // 16-byte chunks per row
  constexpr int TPI = 64 / CPR;
  constexpr int NB = 8;
  const int n_inst = (n + TPI - 1) / TPI;
  const int my_t = lane / CPR, my_c = lane % CPR;
  const Rsrc rs = make_rsrc(rows, uint32_t(n) * D * 2);
  uint32_t qq[GQ][4];
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    const uint4 x = h < nh ? reinterpret_cast<const uint4*>(qg + h * D)[my_c] : make_uint4(0, 0, 0, 0);
    const half2_t s8 = as_h2(0x1C001C00u);                        // * 2^-8, exact
    qq[h][0] = as_u32(as_h2(x.x) * s8);
    qq[h][1] = as_u32(as_h2(x.y) * s8);
    qq[h][2] = as_u32(as_h2(x.z) * s8);
    qq[h][3] = as_u32(as_h2(x.w) * s8);
  }
  const uint32_t lane_off = uint32_t((my_t * D + my_c * 8) * 2);
  for (int i0 = 0; i0 < n_inst; i0 += NB) {
    uint4 buf[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) buf[u] = bload<4>(rs, lane_off + uint32_t((i0 + u) * TPI * D * 2));
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int i = i0 + u;
      if (i >= n_inst) continue;
      const uint4 x = buf[u];
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        float acc = dot2(qq[h][0], x.x, 0.f);
        acc = dot2(qq[h][1], x.y, acc);
        acc = dot2(qq[h][2], x.z, acc);
        acc = dot2(qq[h][3], x.w, acc);
        W.logit[h * LT + slot0 + i * TPI + my_t] = group_sum<CPR>(acc);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Cross-lane reduction of value partials.  Lane l holds x[0..NX) for chunk
// c = l % CPL; lanes with equal l % CPL are summed.  Within each row of 16
// lanes the sums come from DPP rotations; the four rows' sums are left in
// W.red as red[(row * CPL + c) * NX + j].
template <int CPL, int NX>
__device__ __forceinline__ void reduce_rows(const WaveLds& W, float (&x)[NX], int lane) {
#pragma unroll
  for (int j = 0; j < NX; ++j) {
    float y = x[j];
    if (CPL <= 8) y = row_ror_add<8>(y);
    if (CPL <= 4) y = row_ror_add<4>(y);
    if (CPL <= 2) y = row_ror_add<2>(y);
    if (CPL <= 1) y = row_ror_add<1>(y);
    x[j] = y;
  }
  // lanes (lane % 16) < CPL now hold their row's sums
  float* red = W.red;
  const int row = lane >> 4, c = lane & 15;
  if (c < CPL) {
#pragma unroll
    for (int j = 0; j < NX; ++j) red[(row * CPL + c) * NX + j] = x[j];
  }
  wave_lds_sync();
}

// Values of run tokens [r0, r1) (bits 2/4/8); cbase / mbase address the run's
// pair block 0 (codes and meta) of this stream.  Pair block p of the run holds
// run tokens 2p and 2p+1, whose probabilities are fp16 pair p - r0/2 of W.p16
// counted from dword ps0 (r0 is even).  Slot ph >= 0 (the partner after an
// odd run's last token, a token of the next piece) reads as zero while the
// run is read; the partner's meta is finite.  Pair blocks past the range read
// zero codes and zero meta, so they add 0.  Unless softmax_done, `softmax`
// runs after the first loads are issued (it writes W.p16).
template <int D, int GQ, int BITS, class Softmax, bool PG = false>
__device__ __forceinline__ void values_quantized(const DecodeParams& P, const WaveLds& W,
                                 const uint8_t* cbase, const uint8_t* mbase, int r0, int r1, int ps0, int lane,
                                 Softmax& softmax, bool softmax_done, int ph, int n_wave, PageLoc* loc = nullptr) {
  constexpr int LT = wave_slots(GQ);
  constexpr int RB = D * BITS / 8;
  constexpr int CPP = 2 * RB / 16;        // 16-byte chunks per pair block
  constexpr int PPI = 64 / CPP;           // pair blocks per wave instruction
  constexpr int CPCV = 64 / BITS;         // channels per chunk
  using UP = Unpacker<BITS, true>;        // offsets up to 1024, fewer shifts
  constexpr int NP = UP::NP;              // channels per 16-bit unit
  const UP unpack;                        // constants in registers, once
  // heads per pass over the values: every head at once up to 4 heads (their
  // accumulators fit the two-waves-per-SIMD register budget), so the codes
  // are read and unpacked once
  constexpr int HPP = GQ <= 4 ? GQ : (64 / CPCV > 1 ? 64 / CPCV : 1);
  constexpr int NBV = value_batch<GQ>();
  constexpr int NX = CPCV + 2;
  const int NG = D >> P.lg_g;
  const int my_p = lane / CPP, my_c = lane % CPP;
  const int g = (my_c * CPCV) >> P.lg_g;
  const int p0 = r0 >> 1;
  const int np = ((r1 - 1) >> 1) - p0 + 1;
  const int n_inst = (np + PPI - 1) / PPI;
  // (paged: the page cursor supplies the buffers; cbase and mbase are null)
  const Rsrc crs = make_rsrc(cbase + (PG ? 0 : int64_t(p0) * 2 * RB), PG ? 0u : uint32_t(np) * 2 * RB);
  const Rsrc mrs = make_rsrc(mbase + (PG ? 0 : int64_t(p0) * NG * 8), PG ? 0u : uint32_t(np) * NG * 8);
  const uint32_t c_off = uint32_t(my_p * 2 * RB + my_c * 16);
  const uint32_t m_off = uint32_t((my_p * NG + g) * 8);
  const uint32_t* pp = reinterpret_cast<const uint32_t*>(W.p16) + ps0;
  const half2_t one2 = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
  static_assert(!PG || HPP == GQ, "the page cursor moves forward only: one pass");

  uint16_t keep[GQ];
  for (int hp = 0; hp < GQ; hp += HPP) {
    float acc[HPP][NX];                   // [CPCV] channel sums, then sum(p*s), sum(p*z)
#pragma unroll
    for (int hh = 0; hh < HPP; ++hh)
#pragma unroll
      for (int j = 0; j < NX; ++j) acc[hh][j] = 0.f;
    // software pipeline as in keys_quantized: batch b+1 in flight while b is
    // consumed; batches past the end read zeros and touch no memory
    struct Batch {
      uint4 cb[NBV];
      uint2 mb[NBV];
    };
    auto issue = [&](Batch& B, int i0) {
      if constexpr (PG) {
        // an instruction's 32 tokens lie in one page
        const int t = r0 + 2 * i0 * PPI;
        loc->at(t);
#pragma unroll
        for (int u = 0; u < NBV; ++u) {
          uint32_t oc, om;
          const Rsrc rc = loc->code(t + 2 * u * PPI, oc);
          const Rsrc rm = loc->meta(t + 2 * u * PPI, om);
          B.cb[u] = bload<4>(rc, oc + c_off);
          B.mb[u] = bload<2>(rm, om + m_off);
        }
      } else {
#pragma unroll
        for (int u = 0; u < NBV; ++u) {
          B.cb[u] = bload<4>(crs, c_off + uint32_t((i0 + u) * PPI * 2 * RB));
          B.mb[u] = bload<2>(mrs, m_off + uint32_t((i0 + u) * PPI * NG * 8));
        }
      }
    };
    auto consume = [&](const Batch& B, int i0) {
#pragma unroll
      for (int u = 0; u < NBV; ++u) {
        if (i0 + u >= n_inst) continue;     // uniform
        const half2_t s2 = as_h2(__builtin_amdgcn_perm(B.mb[u].y, B.mb[u].x, 0x05040100u));
        const half2_t z2 = as_h2(__builtin_amdgcn_perm(B.mb[u].y, B.mb[u].x, 0x07060302u));
        uint32_t ps[HPP];
#pragma unroll
        for (int hh = 0; hh < HPP; ++hh) {
          // pairs past the range hold probabilities of later slots or zeros
          // (finite) against meta that reads as zero; with more than 16
          // pairs per instruction they could pass the wave's slots, so pair
          // np (a zero slot, or a probability of the next piece) stands in
          const int pi = (i0 + u) * PPI + my_p;
          const half2_t p2 = as_h2(pp[(hp + hh) * (LT / 2) + (PPI > 16 ? min(pi, np) : pi)]);
          const half2_t psh = p2 * s2;
          ps[hh] = as_u32(psh);
          acc[hh][CPCV] = __builtin_amdgcn_fdot2(psh, one2, acc[hh][CPCV], false);
          acc[hh][CPCV + 1] = __builtin_amdgcn_fdot2(p2, z2, acc[hh][CPCV + 1], false);
        }
        // one word at a time: unpack, then apply it to every head
        const uint32_t words[4] = {B.cb[u].x, B.cb[u].y, B.cb[u].z, B.cb[u].w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t v[NP];
          unpack.run(words[w], v);
#pragma unroll
          for (int hh = 0; hh < HPP; ++hh)
#pragma unroll
            for (int k = 0; k < NP; ++k) acc[hh][w * NP + k] = dot2(ps[hh], v[k], acc[hh][w * NP + k]);
        }
      }
    };
    Batch A, Bb;
    issue(A, 0);
    if (hp == 0) {
      // the probabilities are made while the first loads are in flight
      if (!softmax_done) softmax();
      if (ph >= 0) {
        // (uniform) clear the partner slot after an odd run end for this run
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
          keep[h] = W.p16[h * LT + ph];
          wave_lds_sync();
          if (lane == 0) W.p16[h * LT + ph] = 0;
        }
        wave_lds_sync();
      }
    }
    for (int i0 = 0; i0 < n_inst; i0 += 2 * NBV) {
      progress_prio(1, 2 * (ps0 + i0 * PPI), n_wave);
      issue(Bb, i0 + NBV);
      consume(A, i0);
      issue(A, i0 + 2 * NBV);
      if (i0 + NBV < n_inst) consume(Bb, i0 + NBV);
    }
#pragma unroll
    for (int hh = 0; hh < HPP; ++hh) {
      reduce_rows<CPP, NX>(W, acc[hh], lane);
      const float* red = W.red;
#pragma unroll
      for (int k = 0; k < D / 64; ++k) {
        const int ch = lane + 64 * k;
        const int c = ch / CPCV, j = ch % CPCV;
        float a = 0.f, s = 0.f, z = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float* e = red + (r * CPP + c) * NX;
          a += e[j];
          s += e[CPCV];
          z += e[CPCV + 1];
        }
        W.ow[(hp + hh) * (D + 2) + 2 + ch] += a - UP::offset(j % NP) * s + z;
      }
      wave_lds_sync();
    }
  }
  if (ph >= 0) {
#pragma unroll
    for (int h = 0; h < GQ; ++h)
      if (lane == 0) W.p16[h * LT + ph] = keep[h];
    wave_lds_sync();
  }
}

// The same values on matrix cores, for d_h = 128 and grouped query heads:
// the A.V products of every head come from v_mfma_f32_16x16x32_f16, so the
// code unpacking is the only per-element work and is shared by the heads.
//
// A step is 16 pair blocks (32 tokens).  Lane l is column n = l % 16 and
// k-block kb = l / 16 of the operands: it reads bytes [n LW, (n+1) LW) of
// pair blocks 4 kb .. 4 kb + 3 (LW = 2 RB / 16, one 4, 8 or 16-byte load
// each: channels 8n .. 8n+7 of both tokens), so every k-block row of 16
// lanes holds the same eight tokens.  B of instruction j is channel 8n + j
// of those tokens, unpacked as (offset + code) pairs; A row m is (head
// m >> lg(NG), channel group m & (NG - 1)) with NG = 128 / G groups per
// token, and holds p * s of that head and group for the eight tokens (fp16,
// as in the pair loop above), so D row (h, g) at column n is
//   sum_t p_h(t) s_g(t) (offset_j + code_t,8n+j),
// which is wanted where 8n + j lies in group g.  Up to 16 / NG heads share an
// A block; more heads take a second block against the same B.  sum p * s and
// sum p * z of each row are kept beside, summed over the four k-blocks at
// the end and folded in: o = D - offset_j sum(p s) + sum(p z).
template <int D, int GQ, int BITS, class Softmax, bool PG = false>
__device__ __forceinline__ void values_quantized_mfma(int lg_g, const WaveLds& W,
                                      const uint8_t* cbase, const uint8_t* mbase, int r0, int r1, int ps0, int lane,
                                      Softmax& softmax, bool softmax_done, int ph, int n_wave,
                                      PageLoc* loc = nullptr) {
  static_assert(D == 128, "eight channels per lane and column");
  constexpr int LT = wave_slots(GQ);
  constexpr int RB = D * BITS / 8;
  constexpr int LW = 2 * RB / 16;         // bytes per lane and pair block
  constexpr int WPL = LW / 4;
  using UP = Unpacker<BITS, true>;
  constexpr int NP = UP::NP;              // channels per word
  static_assert(WPL * NP == 8, "eight channels per lane");
  constexpr int NAB = (GQ + 3) / 4;       // A blocks for 32-channel groups
  constexpr int NBV = BITS == 2 ? 2 : 1;  // steps per load batch
  const UP unpack;
  const int lg_ng = 7 - lg_g;
  const int NG = 1 << lg_ng;
  const int hpb = 16 >> lg_ng;            // heads per A block
  const int nab = (GQ + hpb - 1) / hpb;   // (uniform) A blocks in use
  const int col = lane & 15, kb = lane >> 4;
  const int ga = col & (NG - 1);          // the group of the lane's A row
  const int p0 = r0 >> 1;
  const int np = ((r1 - 1) >> 1) - p0 + 1;
  const int n_steps = (np + 15) >> 4;
  // (paged: the page cursor supplies the buffers; cbase and mbase are null)
  const Rsrc crs = make_rsrc(cbase + (PG ? 0 : int64_t(p0) * 2 * RB), PG ? 0u : uint32_t(np) * 2 * RB);
  const Rsrc mrs = make_rsrc(mbase + (PG ? 0 : int64_t(p0) * NG * 8), PG ? 0u : uint32_t(np) * NG * 8);
  const uint32_t c_off = uint32_t(4 * kb * 2 * RB + col * LW);
  const uint32_t m_off = uint32_t((4 * kb * NG + ga) * 8);
  const uint32_t* pp = reinterpret_cast<const uint32_t*>(W.p16) + ps0;
  const half2_t one2 = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
  // the lane's p16 pairs: the row of its A-row head (padded rows repeat a
  // head) from the first pair of its k-block
  const uint32_t* prow[NAB];
#pragma unroll
  for (int ab = 0; ab < NAB; ++ab) prow[ab] = pp + min(ab * hpb + (col >> lg_ng), GQ - 1) * (LT / 2) + 4 * kb;

  float4_t acc[NAB][8];
  float srow[NAB], zrow[NAB];
#pragma unroll
  for (int ab = 0; ab < NAB; ++ab) {
    srow[ab] = 0.f;
    zrow[ab] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[ab][j] = float4_t{0.f, 0.f, 0.f, 0.f};
  }
  // steps past the end read zeros and touch no memory
  struct Batch {
    typename LoadType<WPL>::T c[NBV][4];
    uint2 m[NBV][4];
  };
  auto issue = [&](Batch& B, int s0) {
    if constexpr (PG) {
      // a step's 32 tokens lie in one page
      loc->at(r0 + 32 * s0);
#pragma unroll
      for (int v = 0; v < NBV; ++v) {
        uint32_t oc, om;
        const Rsrc rc = loc->code(r0 + 32 * (s0 + v), oc);
        const Rsrc rm = loc->meta(r0 + 32 * (s0 + v), om);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          B.c[v][u] = bload<WPL>(rc, oc + c_off + uint32_t(u * 2 * RB));
          B.m[v][u] = bload<2>(rm, om + m_off + uint32_t(u * NG * 8));
        }
      }
    } else {
#pragma unroll
      for (int v = 0; v < NBV; ++v)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int pr = 16 * (s0 + v) + u;
          B.c[v][u] = bload<WPL>(crs, c_off + uint32_t(pr * 2 * RB));
          B.m[v][u] = bload<2>(mrs, m_off + uint32_t(pr * NG * 8));
        }
    }
  };
  auto consume = [&](const Batch& B, int s0) {
#pragma unroll
    for (int v = 0; v < NBV; ++v) {
      if (s0 + v >= n_steps) continue;    // uniform
      const int pb = 16 * (s0 + v);       // the step's first pair
      uint32_t s2[4], z2[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        s2[u] = __builtin_amdgcn_perm(B.m[v][u].y, B.m[v][u].x, 0x05040100u);
        z2[u] = __builtin_amdgcn_perm(B.m[v][u].y, B.m[v][u].x, 0x07060302u);
      }
      half8_t am[NAB];
#pragma unroll
      for (int ab = 0; ab < NAB; ++ab) {
        if (ab >= nab) continue;          // uniform
        uint32_t aw[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          // pairs past the range (at most 15, within the wave's slots) hold
          // probabilities of later slots or zeros, finite, against meta that
          // reads as zero
          const half2_t p2 = as_h2(prow[ab][pb + u]);
          const half2_t psh = p2 * as_h2(s2[u]);
          aw[u] = as_u32(psh);
          srow[ab] = __builtin_amdgcn_fdot2(psh, one2, srow[ab], false);
          zrow[ab] = __builtin_amdgcn_fdot2(p2, as_h2(z2[u]), zrow[ab], false);
        }
        am[ab] = __builtin_bit_cast(half8_t, make_uint4(aw[0], aw[1], aw[2], aw[3]));
      }
      uint32_t vv[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < WPL; ++w) unpack.run(word<WPL>(B.c[v][u], w), &vv[u][w * NP]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const half8_t bm = __builtin_bit_cast(half8_t, make_uint4(vv[0][j], vv[1][j], vv[2][j], vv[3][j]));
#pragma unroll
        for (int ab = 0; ab < NAB; ++ab)
          if (ab < nab) acc[ab][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(am[ab], bm, acc[ab][j], 0, 0, 0);
      }
    }
  };

  Batch A, Bb, Cc;
  issue(A, 0);
  if constexpr (stream_batches<D, GQ>() == 3) issue(Bb, NBV);
  uint16_t keep[GQ];
  // the probabilities are made while the first loads are in flight
  if (!softmax_done) softmax();
  if (ph >= 0) {
    // (uniform) clear the partner slot after an odd run end for this run
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      keep[h] = W.p16[h * LT + ph];
      wave_lds_sync();
      if (lane == 0) W.p16[h * LT + ph] = 0;
    }
    wave_lds_sync();
  }
  if constexpr (stream_batches<D, GQ>() == 3) {
    for (int s0 = 0; s0 < n_steps; s0 += 3 * NBV) {
      progress_prio(1, 2 * (ps0 + 16 * s0), n_wave);
      issue(Cc, s0 + 2 * NBV);
      consume(A, s0);
      issue(A, s0 + 3 * NBV);
      if (s0 + NBV < n_steps) consume(Bb, s0 + NBV);
      issue(Bb, s0 + 4 * NBV);
      if (s0 + 2 * NBV < n_steps) consume(Cc, s0 + 2 * NBV);
    }
  } else {
    for (int s0 = 0; s0 < n_steps; s0 += 2 * NBV) {
      progress_prio(1, 2 * (ps0 + 16 * s0), n_wave);
      issue(Bb, s0 + NBV);
      consume(A, s0);
      issue(A, s0 + 2 * NBV);
      if (s0 + NBV < n_steps) consume(Bb, s0 + NBV);
    }
  }

  // row sums over the four k-blocks, then to LDS
  float* red = W.red;                     // [NAB][sum p*s of 16 rows | sum p*z of 16 rows]
#pragma unroll
  for (int ab = 0; ab < NAB; ++ab) {
    float x = srow[ab], y = zrow[ab];
    auto a1 = __builtin_amdgcn_permlane16_swap(fbits(x), fbits(x), false, false);
    auto b1 = __builtin_amdgcn_permlane16_swap(fbits(y), fbits(y), false, false);
    x = bitsf(a1[0]) + bitsf(a1[1]);
    y = bitsf(b1[0]) + bitsf(b1[1]);
    auto a2 = __builtin_amdgcn_permlane32_swap(fbits(x), fbits(x), false, false);
    auto b2 = __builtin_amdgcn_permlane32_swap(fbits(y), fbits(y), false, false);
    x = bitsf(a2[0]) + bitsf(a2[1]);
    y = bitsf(b2[0]) + bitsf(b2[1]);
    if (lane < 16) {
      red[ab * 32 + col] = x;
      red[ab * 32 + 16 + col] = y;
    }
  }
  wave_lds_sync();
  // lane (n, kb) holds D rows 4 kb .. 4 kb + 3 at column n for channels
  // 8n .. 8n+7, all in group gc
  const int gc = (8 * col) >> lg_g;
#pragma unroll
  for (int ab = 0; ab < NAB; ++ab) {
    if (ab >= nab) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * kb + r;
      const int h = ab * hpb + (row >> lg_ng);
      if ((row & (NG - 1)) != gc || h >= GQ) continue;
      const float sr = red[ab * 32 + row], zr = red[ab * 32 + 16 + row];
      float* o = W.ow + h * (D + 2) + 2 + 8 * col;
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] += acc[ab][j][r] - UP::offset(j % NP) * sr + zr;
    }
  }
  wave_lds_sync();
  if (ph >= 0) {
#pragma unroll
    for (int h = 0; h < GQ; ++h)
      if (lane == 0) W.p16[h * LT + ph] = keep[h];
    wave_lds_sync();
  }
}

// Quantized values: matrix cores for grouped heads at d_h = 128, the pair
// loop otherwise.
template <int D, int GQ, int BITS, bool PG = false, class Softmax>
__device__ __forceinline__ void values_q(const DecodeParams& P, const WaveLds& W, const uint8_t* cbase,
                                         const uint8_t* mbase, int r0, int r1, int ps0, int lane, Softmax& softmax,
                                         bool softmax_done, int ph, int n_wave, PageLoc* loc = nullptr) {
  if constexpr (D == 128 && GQ >= 2)
    values_quantized_mfma<D, GQ, BITS, Softmax, PG>(P.lg_g, W, cbase, mbase, r0, r1, ps0, lane, softmax,
                                                    softmax_done, ph, n_wave, loc);
  else
    values_quantized<D, GQ, BITS, Softmax, PG>(P, W, cbase, mbase, r0, r1, ps0, lane, softmax, softmax_done, ph,
                                               n_wave, loc);
}

// Values from fp16 rows rows[0..n), probabilities at slots slot0 + i
// (slots past the range are zero or belong to other pieces; rows past the
// range read as zero).
template <int D, int GQ>
__device__ __forceinline__ void values_fp16(const DecodeParams& P, const WaveLds& W, const uint16_t* rows,
                            int n, int slot0, int lane) {
  constexpr int LT = wave_slots(GQ);
  constexpr int CPR = D / 8;
  constexpr int TPI = 64 / CPR;
  constexpr int NB = 8;
  const int my_t = lane / CPR, my_c = lane % CPR;
  const int n_inst = (n + TPI - 1) / TPI;
  const Rsrc rs = make_rsrc(rows, uint32_t(n) * D * 2);
  const uint32_t lane_off = uint32_t((my_t * D + my_c * 8) * 2);
  float acc[GQ][8];
#pragma unroll
  for (int h = 0; h < GQ; ++h)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[h][j] = 0.f;
  for (int i0 = 0; i0 < n_inst; i0 += NB) {
    uint4 buf[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) buf[u] = bload<4>(rs, lane_off + uint32_t((i0 + u) * TPI * D * 2));
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int t = (i0 + u) * TPI + my_t;
      const uint4 x = buf[u];
      const uint32_t wv[4] = {x.x, x.y, x.z, x.w};
      float f[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[2 * e] = h2f(wv[e] & 0xffffu);
        f[2 * e + 1] = h2f(wv[e] >> 16);
      }
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        const float p = t < n ? h2f(W.p16[h * LT + slot0 + t]) : 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] += p * f[j];
      }
    }
  }
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    reduce_rows<CPR, 8>(W, acc[h], lane);
    const float* red = W.red;
#pragma unroll
    for (int k = 0; k < D / 64; ++k) {
      const int ch = lane + 64 * k;
      const int c = ch / 8, j = ch % 8;
      float a = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) a += red[(r * CPR + c) * 8 + j];
      W.ow[h * (D + 2) + 2 + ch] += a;
    }
    wave_lds_sync();
  }
}

// ---------------------------------------------------------------------------
// Four waves per SIMD (<= 128 VGPRs) for one query head per kv head: 16
// resident waves per CU (two workgroups) keep enough loads in flight to
// cover HBM latency.  Grouped heads do GQ times the arithmetic per byte:
// two heads get 256 VGPRs (one 8-wave workgroup per CU), head blocks of 4
// three waves per SIMD at 168 VGPRs (one 12-wave workgroup per CU).
template <int D, int GQ, int NW, bool PAGED>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(decode_waves_per_simd(D, GQ))))
decode_kernel(const DecodeParams P) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int LT = wave_slots(GQ);
  constexpr int DK = D / 64;
  constexpr DecodeLds lay = decode_lds<D, GQ>();
  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform (scalar) so that every loop bound derived from it is scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int wg = blockIdx.x;
  int64_t stream = blockIdx.y;
  if constexpr (PAGED) {
    if (P.sched_n > 0) {
      // 1-D grid in the host's order: find the sequence that owns this workgroup
      const int i = int(blockIdx.x);
      int lo = 0, hi = P.sched_n - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (P.sched_start[mid] <= i) lo = mid;
        else hi = mid - 1;
      }
      const int per = (P.sched_start[lo + 1] - P.sched_start[lo]) / P.Hkv;   // workgroups per stream
      const int j = i - P.sched_start[lo];
      stream = int64_t(P.sched_seq[lo]) * P.Hkv + j / per;
      wg = j % per;
    }
  }
  const int b = int(stream / P.Hkv), hkv = int(stream % P.Hkv);
  const int gw = wg * NW + wave;
  int N, n_kq, n_vq, a, e;
  if constexpr (PAGED) {
    // this sequence's lengths; workgroups past the stream's share leave at once
    n_kq = P.lens[4 * b];
    n_vq = P.lens[4 * b + 1];
    N = n_kq + P.lens[4 * b + 2];
    const PagedCost pc = paged_cost(D, P.G, P.bits);
    const int nwg = paged_wgs(pc, n_kq, n_vq, N, P.pg_wave_tokens, NW);
    if (wg >= nwg) return;                   // the whole workgroup, before any barrier
    a = paged_bound(pc, n_kq, n_vq, N, gw, nwg * NW);
    e = paged_bound(pc, n_kq, n_vq, N, gw + 1, nwg * NW);
  } else {
    N = P.n_tok;
    n_kq = P.n_kq;
    n_vq = P.n_vq;
    const bool tab = P.n_bounds > 0;
    a = tab ? P.bounds[gw] : wave_bound(P.pieces, P.n_pieces, P.cost_total, N, gw, P.waves_per_stream);
    e = tab ? P.bounds[gw + 1] : wave_bound(P.pieces, P.n_pieces, P.cost_total, N, gw + 1, P.waves_per_stream);
  }
  const int n = e - a;

  // query heads h0 .. h0 + nh - 1 of the kv head's gq (head block blockIdx.z
  // of GQ heads; more than GQ heads per kv head take several blocks)
  const int h0 = int(blockIdx.z) * GQ;
  const int nh = min(GQ, P.gq - h0);
  const uint16_t* qg = P.q + (int64_t(b) * P.Hq + int64_t(hkv) * P.gq + h0) * D;   // [nh][D]

  if (!PAGED && P.fused_append && wave == NW - 1) {
    // this stream's decode-step append, by the wave whose range holds every
    // token it writes; its stores complete before the wave reads them
    const AppendParams& ap = P.app;
    switch (ap.bits * 1000 + ap.G) {
      case 2032: append_stream<2, D, 32>(ap, stream, lane); break;
      case 2064: append_stream<2, D, 64>(ap, stream, lane); break;
      case 4032: append_stream<4, D, 32>(ap, stream, lane); break;
      case 4064: append_stream<4, D, 64>(ap, stream, lane); break;
      case 8032: append_stream<8, D, 32>(ap, stream, lane); break;
      case 8064: append_stream<8, D, 64>(ap, stream, lane); break;
      default:
        if constexpr (D >= 128) {
          switch (ap.bits) {
            case 2: append_stream<2, D, (D >= 128 ? 128 : 64)>(ap, stream, lane); break;
            case 4: append_stream<4, D, (D >= 128 ? 128 : 64)>(ap, stream, lane); break;
            default: append_stream<8, D, (D >= 128 ? 128 : 64)>(ap, stream, lane); break;
          }
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }

  const WaveLds W = carve_wave<D, GQ>(smem, wave);
  // token t of the wave sits at slot t - a; a is even and quantized value
  // runs start at even tokens, so every value pair block starts at an even slot
  if (n > 0) {
    // key pieces in token order
    if constexpr (PAGED && D == 128) {
      // quantized keys: one load pipeline across the pages of the range (a
      // range inside one page takes the plain run loop)
      const int kend = min(e, n_kq);
      if (a < kend && a / P.page_tokens == (kend - 1) / P.page_tokens) {
        const int pg = a / P.page_tokens;
        const int p0 = pg * P.page_tokens;
        const uint8_t* hb = P.pages + int64_t(P.block_table[int64_t(b) * P.max_pages + pg]) * P.page_bytes +
                            int64_t(hkv) * P.head_bytes;
        switch (P.bits) {
          case 2: keys_q<D, GQ, 2>(P, W, qg, nh, hb, hb + P.pg_kmeta_off, a - p0, kend - p0, 0, lane, n); break;
          case 4: keys_q<D, GQ, 4>(P, W, qg, nh, hb, hb + P.pg_kmeta_off, a - p0, kend - p0, 0, lane, n); break;
          default: keys_q<D, GQ, 8>(P, W, qg, nh, hb, hb + P.pg_kmeta_off, a - p0, kend - p0, 0, lane, n); break;
        }
      } else if (a < kend) {
        PageLoc loc;
        loc.head = P.pages + int64_t(hkv) * P.head_bytes;
        loc.page_bytes = P.page_bytes;
        loc.PT = P.page_tokens;
        loc.c_off = 0;
        loc.m_off = P.pg_kmeta_off;
        loc.n_valid = n_kq;
        loc.lg_cu = 0;
        loc.cu_bytes = D * P.bits / 8;
        loc.lg_mu = P.lg_g;
        loc.mu_bytes = D * 4;
        loc.start(P.block_table + int64_t(b) * P.max_pages, P.max_pages, a, lane);
        switch (P.bits) {
          case 2: keys_q<D, GQ, 2, true>(P, W, qg, nh, nullptr, nullptr, a, kend, 0, lane, n, &loc); break;
          case 4: keys_q<D, GQ, 4, true>(P, W, qg, nh, nullptr, nullptr, a, kend, 0, lane, n, &loc); break;
          default: keys_q<D, GQ, 8, true>(P, W, qg, nh, nullptr, nullptr, a, kend, 0, lane, n, &loc); break;
        }
      }
    } else if constexpr (PAGED) {
      // quantized keys, one piece per page (pages start on key groups)
      const int kend = min(e, n_kq);
      for (int t0 = a; t0 < kend;) {
        const int pg = t0 / P.page_tokens;
        const int p0 = pg * P.page_tokens;
        const int t1 = min(kend, p0 + P.page_tokens);
        const uint8_t* hb = P.pages + int64_t(P.block_table[int64_t(b) * P.max_pages + pg]) * P.page_bytes +
                            int64_t(hkv) * P.head_bytes;
        switch (P.bits) {
          case 2: keys_q<D, GQ, 2>(P, W, qg, nh, hb, hb + P.pg_kmeta_off, t0 - p0, t1 - p0, t0 - a, lane, n); break;
          case 4: keys_q<D, GQ, 4>(P, W, qg, nh, hb, hb + P.pg_kmeta_off, t0 - p0, t1 - p0, t0 - a, lane, n); break;
          default: keys_q<D, GQ, 8>(P, W, qg, nh, hb, hb + P.pg_kmeta_off, t0 - p0, t1 - p0, t0 - a, lane, n); break;
        }
        t0 = t1;
      }
    }
    for (int k = 0; k < (PAGED ? 0 : P.n_k_runs); ++k) {
      const Run& run = P.k_runs[k];
      const int t0 = max(a, run.tok_begin), t1 = min(e, run.tok_begin + run.n_tok);
      if (t0 >= t1) continue;
      const int r0 = t0 - run.tok_begin, r1 = t1 - run.tok_begin;
      const uint8_t* cb = P.k_codes + stream * P.k_codes_stride + run.code_off;
      const uint8_t* mb = P.k_meta + stream * P.k_meta_stride + run.meta_off;
      switch (run.bits) {
        case 2: keys_q<D, GQ, 2>(P, W, qg, nh, cb, mb, r0, r1, t0 - a, lane, n); break;
        case 4: keys_q<D, GQ, 4>(P, W, qg, nh, cb, mb, r0, r1, t0 - a, lane, n); break;
        case 8: keys_q<D, GQ, 8>(P, W, qg, nh, cb, mb, r0, r1, t0 - a, lane, n); break;
        default:
          keys_fp16<D, GQ>(P, W, qg, nh,
                           reinterpret_cast<const uint16_t*>(P.k_codes + stream * P.k_codes_stride + run.code_off) +
                               int64_t(r0) * D,
                           r1 - r0, t0 - a, lane);
      }
    }
    if (e > n_kq) {
      const int t0 = max(a, n_kq);
      keys_fp16<D, GQ>(P, W, qg, nh, P.k_res + stream * P.k_res_stride + int64_t(t0 - n_kq) * D, e - t0,
                       t0 - a, lane);
    }
    wave_lds_sync();
  }

  // softmax state of this wave's range, per head: raw logits x = q'.k, base-2
  // logits x * sc; every slot of p16 is written, zero outside the tokens.
  // It runs once, after the first value piece has issued its first loads
  // (or before any other value piece, or on its own for an empty range).
  float mh[GQ], lh[GQ];
  bool softmax_done = false;
  auto softmax = [&]() {
    const float sc = P.scale_log2 * 256.f;      // undoes q' = q * 2^-8
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      float mx = -INFINITY;
      for (int s = lane * 4; s < n; s += 256) {
        const float4 x = *reinterpret_cast<const float4*>(W.logit + h * LT + s);
        mx = fmaxf(mx, x.x * sc);
        if (s + 1 < n) mx = fmaxf(mx, x.y * sc);
        if (s + 2 < n) mx = fmaxf(mx, x.z * sc);
        if (s + 3 < n) mx = fmaxf(mx, x.w * sc);
      }
      mx = wave_max64(mx);
      const float nm = -mx;
      // exp2 of arguments <= 0 with the bare v_exp_f32: results below the
      // fp32 normal range round to fp16 zero anyway.  Slots past n get 0.
      float sum = 0.f;
#pragma unroll
      for (int s0 = 0; s0 < LT; s0 += 256) {
        const int s = s0 + lane * 4;
        if (s >= LT) continue;
        uint32_t p16[4] = {0u, 0u, 0u, 0u};
        if (s0 < n) {                   // uniform
          const float4 x = *reinterpret_cast<const float4*>(W.logit + h * LT + s);
          const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            if (s + k < n) p16[k] = f2h(__builtin_amdgcn_exp2f(__builtin_fmaf(xs[k], sc, nm)));
            sum += h2f(p16[k]);         // the same rounded values the A.V uses
          }
        }
        *reinterpret_cast<uint2*>(W.p16 + h * LT + s) =
            make_uint2(p16[0] | (p16[1] << 16), p16[2] | (p16[3] << 16));
        // probabilities over the logits: lane l's store lands on logits that
        // other lanes read in this or an earlier step, so no LDS access
        // moves across a step (a wave's LDS accesses run in order)
        if constexpr (p16_over_logits(GQ)) asm volatile("" ::: "memory");
      }
      mh[h] = mx;
      lh[h] = wave_sum64(sum);
    }
    wave_lds_sync();
    softmax_done = true;
  };

  // the wave's output o[D] per head accumulates in its (m, l, o) block, which
  // the value pieces add into (lane l owns channels l + 64k)
#pragma unroll
  for (int h = 0; h < GQ; ++h)
#pragma unroll
    for (int k = 0; k < DK; ++k) W.ow[h * (D + 2) + 2 + lane + 64 * k] = 0.f;
  wave_lds_sync();
  if (n > 0) {
    // value pieces in token order
    if constexpr (PAGED && D == 128) {
      // quantized values: one load pipeline across the pages of the range;
      // an odd end is the last quantized value
      const int vend = min(e, n_vq);
      if (a < vend && a / P.page_tokens == (vend - 1) / P.page_tokens) {
        const int pg = a / P.page_tokens;
        const int p0 = pg * P.page_tokens;
        const uint8_t* hb = P.pages + int64_t(P.block_table[int64_t(b) * P.max_pages + pg]) * P.page_bytes +
                            int64_t(hkv) * P.head_bytes;
        const int ph = ((vend & 1) && vend < e) ? vend - a : -1;
        const uint8_t* cb = hb + P.pg_vcodes_off;
        const uint8_t* mb = hb + P.pg_vmeta_off;
        switch (P.bits) {
          case 2: values_q<D, GQ, 2>(P, W, cb, mb, a - p0, vend - p0, 0, lane, softmax, softmax_done, ph, n); break;
          case 4: values_q<D, GQ, 4>(P, W, cb, mb, a - p0, vend - p0, 0, lane, softmax, softmax_done, ph, n); break;
          default: values_q<D, GQ, 8>(P, W, cb, mb, a - p0, vend - p0, 0, lane, softmax, softmax_done, ph, n); break;
        }
      } else if (a < vend) {
        PageLoc loc;
        loc.head = P.pages + int64_t(hkv) * P.head_bytes;
        loc.page_bytes = P.page_bytes;
        loc.PT = P.page_tokens;
        loc.c_off = P.pg_vcodes_off;
        loc.m_off = P.pg_vmeta_off;
        loc.n_valid = n_vq;
        loc.lg_cu = 1;
        loc.cu_bytes = 2 * D * P.bits / 8;
        loc.lg_mu = 1;
        loc.mu_bytes = (D >> P.lg_g) * 8;
        loc.start(P.block_table + int64_t(b) * P.max_pages, P.max_pages, a, lane);
        const int ph = ((vend & 1) && vend < e) ? vend - a : -1;
        switch (P.bits) {
          case 2: values_q<D, GQ, 2, true>(P, W, nullptr, nullptr, a, vend, 0, lane, softmax, softmax_done, ph, n, &loc); break;
          case 4: values_q<D, GQ, 4, true>(P, W, nullptr, nullptr, a, vend, 0, lane, softmax, softmax_done, ph, n, &loc); break;
          default: values_q<D, GQ, 8, true>(P, W, nullptr, nullptr, a, vend, 0, lane, softmax, softmax_done, ph, n, &loc); break;
        }
      }
    } else if constexpr (PAGED) {
      const int vend = min(e, n_vq);
      for (int t0 = a; t0 < vend;) {
        const int pg = t0 / P.page_tokens;
        const int p0 = pg * P.page_tokens;
        const int t1 = min(vend, p0 + P.page_tokens);
        const uint8_t* hb = P.pages + int64_t(P.block_table[int64_t(b) * P.max_pages + pg]) * P.page_bytes +
                            int64_t(hkv) * P.head_bytes;
        const int r0 = t0 - p0, r1 = t1 - p0;
        // an odd end is the last quantized value (pages hold an even number of tokens)
        const int ph = ((r1 & 1) && t1 < e) ? t1 - a : -1;
        const uint8_t* cb = hb + P.pg_vcodes_off;
        const uint8_t* mb = hb + P.pg_vmeta_off;
        switch (P.bits) {
          case 2: values_q<D, GQ, 2>(P, W, cb, mb, r0, r1, (t0 - a) >> 1, lane, softmax, softmax_done, ph, n); break;
          case 4: values_q<D, GQ, 4>(P, W, cb, mb, r0, r1, (t0 - a) >> 1, lane, softmax, softmax_done, ph, n); break;
          default: values_q<D, GQ, 8>(P, W, cb, mb, r0, r1, (t0 - a) >> 1, lane, softmax, softmax_done, ph, n); break;
        }
        t0 = t1;
      }
    }
    for (int k = 0; k < (PAGED ? 0 : P.n_v_runs); ++k) {
      const Run& run = P.v_runs[k];
      const int t0 = max(a, run.tok_begin), t1 = min(e, run.tok_begin + run.n_tok);
      if (t0 >= t1) continue;
      const int r0 = t0 - run.tok_begin, r1 = t1 - run.tok_begin;
      // the pair partner after an odd run's last token belongs to the next
      // piece: its probability is zero while this run is read
      const int ph = ((r1 & 1) && t1 < e) ? t1 - a : -1;
      const uint8_t* cb = P.v_codes + stream * P.v_codes_stride + run.code_off;
      const uint8_t* mb = P.v_meta + stream * P.v_meta_stride + run.meta_off;
      switch (run.bits) {
        case 2: values_q<D, GQ, 2>(P, W, cb, mb, r0, r1, (t0 - a) >> 1, lane, softmax, softmax_done, ph, n); break;
        case 4: values_q<D, GQ, 4>(P, W, cb, mb, r0, r1, (t0 - a) >> 1, lane, softmax, softmax_done, ph, n); break;
        case 8: values_q<D, GQ, 8>(P, W, cb, mb, r0, r1, (t0 - a) >> 1, lane, softmax, softmax_done, ph, n); break;
        default:
          if (!softmax_done) softmax();
          values_fp16<D, GQ>(P, W,
                             reinterpret_cast<const uint16_t*>(P.v_codes + stream * P.v_codes_stride + run.code_off) +
                                 int64_t(r0) * D,
                             r1 - r0, t0 - a, lane);
      }
    }
    if (e > n_vq) {
      if (!softmax_done) softmax();
      const int t0 = max(a, n_vq);
      values_fp16<D, GQ>(P, W, P.v_res + stream * P.v_res_stride + int64_t(t0 - n_vq) * D, e - t0,
                         t0 - a, lane);
    }
  }
  if (!softmax_done) softmax();
  // the wave's state (an empty wave has m = -inf, l = 0, o = 0)
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      W.ow[h * (D + 2)] = mh[h];
      W.ow[h * (D + 2) + 1] = lh[h];
    }
  }
  __syncthreads();

  // combine the waves; with one workgroup per stream that is the output
  // (and there is no merge kernel)
  const int64_t step = int64_t(P.gq) * (D + 2);
  const bool single = P.wg_per_stream == 1;
  const float* ow0 = reinterpret_cast<const float*>(smem + lay.block + lay.logit + lay.p16);
  constexpr int WSTEP = int(lay.wave / 4);
  for (int i = tid; i < nh * (D + 2); i += NW * 64) {
    const int h = i / (D + 2), j = i % (D + 2);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, ow0[w * WSTEP + h * (D + 2)]);
    float r = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float* ow = ow0 + w * WSTEP + h * (D + 2);
      const float f = ow[0] == M ? 1.f : exp2f(ow[0] - M);   // also -inf == -inf
      r += f * ow[j == 0 ? 1 : j];
      l += f * ow[1];
    }
    if (single) {
      if (j >= 2) P.out[(int64_t(b) * P.Hq + int64_t(hkv) * P.gq + h0 + h) * D + (j - 2)] = r / l;
    } else {
      P.ws[(stream * P.wg_per_stream + wg) * step + int64_t(h0) * (D + 2) + i] = j == 0 ? M : r;
    }
  }
}

// Cross-split merge, one workgroup per (b, hq):
// out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s over the stream's
// workgroup partials, M the largest m_s.  R threads per channel (R * D
// threads, R sized on the host to the partials: one 8-partial chunk per
// thread where that covers them, at most 1024 threads) split the partials;
// each folds its share with a running maximum, CH partials at a time with
// every load of the chunk issued before any is used (one memory round trip
// per chunk, not a max pass and then a sum pass), and the shares of a
// channel meet in LDS.
template <int D, bool PAGED, int R>
__global__ void __launch_bounds__(R * D) merge_kernel(const DecodeParams P) {
  constexpr int MT = R * D;
  constexpr int CH = 8;                      // partials per chunk and thread
  __shared__ float share[3][MT];
  const int tid = threadIdx.x;
  const int64_t bhq = blockIdx.x;
  const int b = int(bhq / P.Hq), hq = int(bhq % P.Hq);
  const int hkv = hq / P.gq, h = hq % P.gq;
  const int64_t stream = int64_t(b) * P.Hkv + hkv;
  const int64_t step = int64_t(P.gq) * (D + 2);
  const float* w0 = P.ws + stream * P.wg_per_stream * step + h * (D + 2);
  int nwg = P.wg_per_stream;
  if constexpr (PAGED) {
    // the workgroups this stream used (the rest of its slots are not written)
    const int n_kq = P.lens[4 * b], n_vq = P.lens[4 * b + 1];
    nwg = paged_wgs(paged_cost(D, P.G, P.bits), n_kq, n_vq, n_kq + P.lens[4 * b + 2], P.pg_wave_tokens,
                    P.waves_per_wg);
  }
  const int c = tid % D, r = tid / D;
  float M = -INFINITY, L = 0.f, O = 0.f;
  for (int s0 = r * CH; s0 < nwg; s0 += R * CH) {
    float m[CH], l[CH], o[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const float* w = w0 + min(s0 + k, nwg - 1) * step;   // past the end: a repeat, skipped below
      m[k] = w[0];
      l[k] = w[1];
      o[k] = w[2 + c];
    }
    float cm = M;
#pragma unroll
    for (int k = 0; k < CH; ++k)
      if (s0 + k < nwg) cm = fmaxf(cm, m[k]);
    const float fr = M == cm ? 1.f : exp2f(M - cm);        // also -inf == -inf
    L *= fr;
    O *= fr;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      if (s0 + k >= nwg) continue;
      const float f = m[k] == cm ? 1.f : exp2f(m[k] - cm);
      L = __builtin_fmaf(l[k], f, L);
      O = __builtin_fmaf(o[k], f, O);
    }
    M = cm;
  }
  if constexpr (R == 1) {
    P.out[bhq * D + c] = O / L;
    return;
  }
  share[0][tid] = M;
  share[1][tid] = L;
  share[2][tid] = O;
  __syncthreads();
  if (r == 0) {
    float Mt = M;
#pragma unroll
    for (int k = 1; k < R; ++k) Mt = fmaxf(Mt, share[0][k * D + c]);
    float Lt = 0.f, Ot = 0.f;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const float mk = share[0][k * D + c];
      const float f = mk == Mt ? 1.f : exp2f(mk - Mt);
      Lt = __builtin_fmaf(share[1][k * D + c], f, Lt);
      Ot = __builtin_fmaf(share[2][k * D + c], f, Ot);
    }
    P.out[bhq * D + c] = Ot / Lt;
  }
}

// the merge with R threads per channel: enough 8-partial chunks for the
// stream with the most workgroups in one round, at most 1024 threads
template <int D, bool PAGED>
hipError_t launch_merge(const DecodeParams& p, hipStream_t s) {
  const dim3 grid(unsigned(int64_t(p.B) * p.Hq));
  const int chunks = (p.wg_per_stream + 7) / 8;
  if (chunks <= 1) hipLaunchKernelGGL((merge_kernel<D, PAGED, 1>), grid, dim3(D), 0, s, p);
  else if (chunks <= 2) hipLaunchKernelGGL((merge_kernel<D, PAGED, 2>), grid, dim3(2 * D), 0, s, p);
  else if (chunks <= 4) hipLaunchKernelGGL((merge_kernel<D, PAGED, 4>), grid, dim3(4 * D), 0, s, p);
  else hipLaunchKernelGGL((merge_kernel<D, PAGED, 1024 / D>), grid, dim3(1024), 0, s, p);
  return hipGetLastError();
}

template <int D, int GQ, int NW, bool PAGED>
hipError_t launch_dgw(const DecodeParams& p, hipStream_t s) {
  const size_t lds = size_t(lds_bytes(decode_lds<D, GQ>(), NW));
  const unsigned hblocks = unsigned((p.gq + GQ - 1) / GQ);
  const dim3 grid = PAGED && p.sched_n > 0 ? dim3(unsigned(p.sched_start[p.sched_n]), 1, hblocks)
                                           : dim3(p.wg_per_stream, p.B * p.Hkv, hblocks);
  hipLaunchKernelGGL((decode_kernel<D, GQ, NW, PAGED>), grid, dim3(NW * 64), lds, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.wg_per_stream == 1) return e;
  return launch_merge<D, PAGED>(p, s);
}

template <int D, int GQ, bool PAGED>
hipError_t launch_dg(const DecodeParams& p, hipStream_t s) {
  if constexpr (GQ == 1 && D == 128)
    if (p.waves_per_wg == kWavesSmall) return launch_dgw<D, GQ, kWavesSmall, PAGED>(p, s);
  if (p.waves_per_wg != decode_waves(D, GQ)) return hipErrorInvalidValue;
  return launch_dgw<D, GQ, decode_waves(D, GQ), PAGED>(p, s);
}

template <int D, bool PAGED>
hipError_t launch_d(const DecodeParams& p, int GQ, hipStream_t s) {
  switch (GQ) {
    case 1: return launch_dg<D, 1, PAGED>(p, s);
    case 2: return launch_dg<D, 2, PAGED>(p, s);
    case 4: return launch_dg<D, 4, PAGED>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int GQ, hipStream_t s) {
  switch (p.D) {
    case 64: return launch_d<64, false>(p, GQ, s);
    case 128: return launch_d<128, false>(p, GQ, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_paged(const DecodeParams& p, int GQ, hipStream_t s) {
  switch (p.D) {
    case 64: return launch_d<64, true>(p, GQ, s);
    case 128: return launch_d<128, true>(p, GQ, s);
    default: return hipErrorInvalidValue;
  }
}

int64_t decode_lds_bytes(int D, int GQ, int waves) {
  switch (D * 16 + GQ) {
    case 64 * 16 + 1: return lds_bytes(decode_lds<64, 1>(), waves);
    case 64 * 16 + 2: return lds_bytes(decode_lds<64, 2>(), waves);
    case 64 * 16 + 4: return lds_bytes(decode_lds<64, 4>(), waves);
    case 128 * 16 + 1: return lds_bytes(decode_lds<128, 1>(), waves);
    case 128 * 16 + 2: return lds_bytes(decode_lds<128, 2>(), waves);
    case 128 * 16 + 4: return lds_bytes(decode_lds<128, 4>(), waves);
    default: return -1;
  }
}

}  // namespace kvq
