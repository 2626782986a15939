// Internal declarations shared by the host entry points (api.hip) and the
// kernel launchers (quantize.hip, reorder.hip, decode.hip).  Not part of the
// ABI: the ABI is include/kvq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kThreads = 256;          // threads per decode / quantize workgroup
constexpr int kWaves = 8;              // waves per decode workgroup
constexpr int kMaxRuns = 8;            // runs per half of the cache
constexpr int kLdsLimit = 160 * 1024;  // LDS of one gfx950 CU: the most a workgroup can use
constexpr int kWaveAlign = 32;         // wave token ranges start at multiples of this
// Query heads per kv head that one decode workgroup serves (its head block):
// 1, 2 or 4; a kv head with more query heads takes several head blocks (grid
// z), each reading the kv head's cache.  A block of 8 heads needs twice the
// LDS per token (the logits and probabilities of 8 heads), which holds its
// waves to 112 tokens and lets the per-wave fixed costs dominate: blocks of 4
// read the cache two to eight times and still ran 1.2-1.6x faster at 7, 8, 16
// and 32 query heads per kv head.
__host__ __device__ constexpr int decode_head_block(int gq) { return gq <= 1 ? 1 : gq <= 2 ? 2 : 4; }
// The PQ scores kernel's head block of gq query heads per kv head (the query
// heads whose tables one workgroup holds): the next power of two, at most 8.
constexpr int kMaxHeadBlock = 8;
__host__ __device__ constexpr int head_block(int gq) {
  return gq <= 1 ? 1 : gq <= 2 ? 2 : gq <= 4 ? 4 : kMaxHeadBlock;
}

// Waves per decode workgroup: 8, or 12 for head blocks of 4 at d_h = 128
// (three waves per SIMD in one workgroup per CU: their registers fit 168
// VGPRs, and their probabilities overwrite the logits, so 12 waves' LDS
// fits 160 KB).
__host__ __device__ constexpr int decode_waves(int D, int GQ) { return GQ >= 4 && D >= 128 ? 12 : kWaves; }
// The 4-wave workgroup of one query head per kv head at d_h = 128 (four per
// CU), for calls with more streams than two 8-wave workgroups per CU hold.
constexpr int kWavesSmall = 4;
// Target tokens per wave; a wave may get up to wave_cap(GQ) tokens.  Larger
// GQ needs more LDS per token (logits and probabilities of GQ heads).  With
// one query head per kv head two workgroups share a CU (48 KB of LDS each);
// grouped heads run one workgroup per CU (their registers), so its waves
// take the longest ranges whose LDS still fits the CU's 160 KB (96 KB at
// d128 for 2 heads, 156 KB for 12 waves of 4 heads): every range restart
// drains a wave's load pipeline, and short waves are all restarts.
__host__ __device__ constexpr int wave_tokens(int GQ) { return GQ <= 2 ? 512 : 320; }
// workgroups per CU of the decode kernel (its register budget)
__host__ __device__ constexpr int decode_wgs_per_cu(int GQ) { return GQ == 1 ? 2 : 1; }
// Head blocks of 4 keep the fp16 probabilities [GQ][LT] in the first half of
// the logit area (each head's softmax writes over logits already consumed)
// and the value reduction's row sums after them.
__host__ __device__ constexpr bool p16_over_logits(int GQ) { return GQ >= 4; }
__host__ __device__ constexpr int wave_cap(int GQ) { return wave_tokens(GQ) * 3 / 2 + kWaveAlign; }
// token slots per wave in LDS: the cap plus 32, since the streaming loops
// read and write whole items (up to 32 tokens) past a range's last token
__host__ __device__ constexpr int wave_slots(int GQ) { return wave_cap(GQ) + 32; }

// Geometry of the quantized-key loop for (D, GQ, BITS).  Logits of 16
// tokens come from D/32 matrix instructions (v_mfma_f32_16x16x32_f16):
// A = the q*s hi and lo rows of the GQ heads (2*GQ of 16 rows), B = the
// tokens' unpacked code pairs (16 columns), k = 32 channels per instruction.
// Lane l holds B column l % 16 for k-block l / 16: it loads LB = RB/4 bytes
// (WPL words, PPL = D/8 code pairs) of one token row, a quarter of it, and
// feeds MF = PPL/4 instructions four pairs each.
template <int D, int GQ, int BITS>
struct KeyGeo {
  static constexpr int RB = D * BITS / 8;       // bytes per token row
  static constexpr int NP = 16 / BITS;          // fp16 code pairs per 32-bit word
  static constexpr int CPW = 32 / BITS;         // channels per 32-bit word
  static constexpr int LB = RB / 4;             // bytes per lane: one k-block of a row
  static constexpr int WPL = LB / 4;            // code words per lane
  static constexpr int PPL = WPL * NP;          // code pairs per lane
  static constexpr int MF = PPL / 4;            // matrix instructions per item
  static constexpr int TPI = 16;                // tokens per item (B columns)
  static constexpr int HD = D / 2;              // code pairs per row
  static constexpr int NB = WPL >= 8 ? 2 : 4;   // items per load batch (two batches in flight)
  static constexpr int NGB = NB * TPI / 32;     // key groups per batch (G >= 32)
  static constexpr int ROWS = 2 * GQ;           // A rows in use: hi and lo of each head
  // LDS dwords per (m, kblock) A block: ROWS rows of 4 dwords plus 4 of
  // padding, so that the 64 lanes' A-row stores of a group (each lane one
  // dword of one block) fall in distinct banks
  static constexpr int BS = ROWS * 4 + 4;
  static constexpr int QBLK = MF * 4 * BS;      // LDS dwords of one group's A blocks [m][kblock][row][4]
  static_assert(PPL * 4 == HD && PPL % 4 == 0, "four k-blocks cover a row, four pairs per instruction");
  static_assert(ROWS <= 16, "at most 8 query heads per head block");
};

__host__ __device__ constexpr int64_t round16(int64_t x) { return (x + 15) / 16 * 16; }
__host__ __device__ constexpr int64_t cmax(int64_t a, int64_t b) { return a > b ? a : b; }

// LDS dwords of the A blocks of one load batch and of the per-(group, head)
// key biases (A blocks are the same size for every code width: D/32
// instructions per item).
template <int D, int GQ>
__host__ __device__ constexpr int64_t kQsMax() {
  return cmax(KeyGeo<D, GQ, 2>::NGB, KeyGeo<D, GQ, 8>::NGB) * KeyGeo<D, GQ, 2>::QBLK;
}
template <int D, int GQ>
__host__ __device__ constexpr int64_t kBiasMax() {
  return cmax(KeyGeo<D, GQ, 2>::NGB, KeyGeo<D, GQ, 8>::NGB) * GQ;
}

// Per-wave LDS of a decode workgroup (the device uses the same numbers).
// Block part: none (q is read from global memory by each wave).  Per
// wave, with LT = wave_slots(GQ):
//   logit  fp32 [GQ][LT]  logits by token slot; reused afterwards for the
//                          row sums of the value reduction (at most 640 floats)
//   p16    fp16 [GQ][LT]  probabilities, zero outside the wave's tokens
//                          (head blocks of 4: over the first half of logit,
//                          the row sums after them)
//   area   A blocks (q*s hi/lo rows) and biases of the key groups of one load batch;
//          afterwards the wave's (m, l, o[D]) per head
struct DecodeLds {
  int64_t block, logit, p16, area, wave, total;   // total: for decode_waves(D, GQ) waves
};
__host__ __device__ constexpr int64_t lds_bytes(const DecodeLds& l, int waves) {
  return l.block + waves * l.wave;
}
template <int D, int GQ>
__host__ __device__ constexpr DecodeLds decode_lds() {
  const int64_t lt = wave_slots(GQ);
  const int64_t block = 0;
  const int64_t logit = round16(cmax(int64_t(GQ) * lt * 4, (p16_over_logits(GQ) ? GQ * lt / 2 : 0) * 4 + 640 * 4));
  const int64_t p16 = p16_over_logits(GQ) ? 0 : round16(int64_t(GQ) * lt * 2);
  // A blocks and zero block, then the per-(group, head) biases (see carve_wave)
  const int64_t qs = (kQsMax<D, GQ>() + kBiasMax<D, GQ>()) * 4;
  const int64_t area = round16(cmax(qs, int64_t(GQ) * (D + 2) * 4));
  const int64_t wave = logit + p16 + area;
  return DecodeLds{block, logit, p16, area, wave, block + decode_waves(D, GQ) * wave};
}

struct Run {            // device copy of kvq_segment
  int32_t bits, tok_begin, n_tok, pad;
  int64_t code_off, meta_off;
};

// Token ranges of uniform HBM cost (bytes per token of keys + values, meta
// included): the cuts of the key and value runs and of the residuals.  Wave
// ranges are cut at equal shares of a stream's cost, so a wave holding fp16
// residual rows (256 bytes per token at d = 128) gets fewer tokens than one
// holding 2-bit codes (about 48).
constexpr int kMaxPieces = 2 * kMaxRuns + 2;
constexpr int kMaxBounds = 64;          // waves per stream with host-computed wave bounds
constexpr int kMaxSched = 256;          // sequences of a paged call with a sorted schedule
struct CostPiece {
  int32_t t0, cost;        // first token, bytes per token
  int64_t c0;              // cost of the tokens before t0
};

// First token of wave range w of nw ranges: the token where the cumulative
// cost reaches w/nw of the total, rounded down to a multiple of kWaveAlign
// (0 for w <= 0, N for w >= nw).  Monotone in w.  nw <= 2^23, so the
// products below stay within 64 bits.
__host__ __device__ inline int wave_bound(const CostPiece* pc, int n_pieces, int64_t total, int N,
                                          int w, int nw) {
  if (w <= 0) return 0;
  if (w >= nw) return N;
  const int64_t target = (total / nw) * w + ((total % nw) * w) / nw;
  int i = 0;
  while (i + 1 < n_pieces && pc[i + 1].c0 <= target) ++i;
  const int64_t t = pc[i].t0 + (target - pc[i].c0) / pc[i].cost;
  const int64_t ta = t & ~int64_t(kWaveAlign - 1);
  return int(ta < N ? ta : N);
}

struct AppendParams {
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_res;
  uint16_t* v_res;
  uint8_t* v_codes;
  uint8_t* v_meta;
  int64_t k_new_stride, v_new_stride, k_res_stride, v_res_stride;   // fp16 elements
  int64_t v_codes_stride, v_meta_stride;                            // bytes
  int32_t bits, G, D, n_streams;
  int32_t k_row, v_row, v_quant_row, v_dst_tok;
};

struct DecodeParams {
  const uint16_t* q;
  float* out;
  float* ws;                            // per-workgroup partials [stream][wg][gq][D+2]
  const uint8_t* k_codes;
  const uint8_t* k_meta;
  const uint8_t* v_codes;
  const uint8_t* v_meta;
  const uint16_t* k_res;
  const uint16_t* v_res;
  int64_t k_codes_stride, k_meta_stride, v_codes_stride, v_meta_stride;
  int64_t k_res_stride, v_res_stride;   // fp16 elements
  int32_t B, Hq, Hkv, D, G, gq;
  int32_t lg_g;                         // log2(G)
  int32_t n_tok;                        // N, tokens attended per stream
  int32_t n_kq, n_vq;                   // tokens held in key runs / value runs
  int32_t waves_per_stream;             // a multiple of waves_per_wg
  int32_t waves_per_wg;                 // decode_waves(D, head block), or kWavesSmall
  int32_t wg_per_stream;
  float scale_log2;                     // sm_scale * log2(e)
  int32_t n_k_runs, n_v_runs;
  Run k_runs[kMaxRuns];
  Run v_runs[kMaxRuns];
  int32_t n_pieces;
  int64_t cost_total;
  CostPiece pieces[kMaxPieces];
  // wave_bound(.., w, waves_per_stream) for w = 0 .. waves_per_stream when
  // waves_per_stream <= kMaxBounds (every stream has the same runs, so the
  // bounds are the same for all of them); otherwise n_bounds = 0 and each
  // wave computes its own (64-bit divisions: ~1 us per launch)
  int32_t n_bounds;
  int32_t bounds[kMaxBounds + 1];
  // fused decode-step append: when set, the last wave of each stream's (only)
  // workgroup first performs that stream's append (app) and then attends over
  // the appended state; the host sets it only when every token the append
  // writes lies in that wave's range
  int32_t fused_append;
  AppendParams app;
  // Paged cache (decode_kernel<..., true>; k_runs, v_runs, pieces and bounds
  // unused).  Sequence b's quantized tokens live in pages of page_tokens
  // tokens: its page j is pool page block_table[b * max_pages + j] at
  // pages + page * page_bytes, kv head h's block at + h * head_bytes, with key
  // codes at 0, key meta at pg_kmeta_off, value codes at pg_vcodes_off and
  // value meta at pg_vmeta_off (the layout of kvq_page_layout).
  // lens[4 b + 0..3] = n_kq, n_vq, n_k_res, n_v_res of sequence b; every
  // stream of the sequence uses paged_wgs(...) of the grid's wg_per_stream
  // workgroups.
  const uint8_t* pages;
  const int32_t* block_table;
  const int32_t* lens;
  int64_t page_bytes, head_bytes;
  int32_t page_tokens, max_pages, pg_kmeta_off, pg_vcodes_off, pg_vmeta_off, bits;
  int32_t pg_wave_tokens;              // paged_wgs's wt (<= wave_cap(GQ) - kWaveAlign)
  // Paged schedule (sched_n > 0, batch <= kMaxSched): a 1-D grid of exactly
  // the workgroups the streams need, heaviest workgroups first.  Sequence
  // sched_seq[k] owns grid workgroups sched_start[k] .. sched_start[k+1]-1:
  // n_kv_heads streams of (sched_start[k+1] - sched_start[k]) / n_kv_heads
  // workgroups each.  sched_n = 0: grid (wg_per_stream, streams), surplus
  // workgroups leave at once.
  int32_t sched_n;
  int32_t sched_start[kMaxSched + 1];
  uint16_t sched_seq[kMaxSched];
};

// Byte costs per token of a paged stream (keys + values): both quantized,
// quantized key + fp16 value, both fp16.
struct PagedCost {
  int32_t both_q, key_q, both_16;
};
__host__ __device__ inline PagedCost paged_cost(int D, int G, int bits) {
  const int32_t rb = D * bits / 8;
  const int32_t kq = rb + D * 4 / G, vq = rb + (D / G) * 4, h16 = 2 * D;
  return PagedCost{kq + vq, kq + h16, 2 * h16};
}
__host__ __device__ inline int64_t paged_total(const PagedCost& c, int n_kq, int n_vq, int N) {
  return int64_t(n_vq) * c.both_q + int64_t(n_kq - n_vq) * c.key_q + int64_t(N - n_kq) * c.both_16;
}
// Workgroups of a paged stream: enough that a wave's share of the stream's
// bytes is at most wt tokens of the cheapest kind; with wt <= wave_cap(GQ) -
// kWaveAlign no wave range exceeds wave_cap(GQ) (the starts are rounded
// down by < kWaveAlign).
__host__ __device__ inline int paged_wgs(const PagedCost& c, int n_kq, int n_vq, int N, int wt, int NW) {
  const int64_t per_wg = int64_t(NW) * wt * c.both_q;
  const int64_t t = paged_total(c, n_kq, n_vq, N);
  const int64_t w = (t + per_wg - 1) / per_wg;
  return int(w < 1 ? 1 : w);
}
// First token of wave range w of nw over a paged stream (same rounding as
// wave_bound): token where the cost reaches w/nw of the total, rounded down
// to a multiple of kWaveAlign.  Monotone in w.
__host__ __device__ inline int paged_bound(const PagedCost& c, int n_kq, int n_vq, int N, int w, int nw) {
  if (w <= 0) return 0;
  if (w >= nw) return N;
  const int64_t total = paged_total(c, n_kq, n_vq, N);
  const int64_t target = total / nw * w + (total % nw) * w / nw;
  const int64_t c0 = int64_t(n_vq) * c.both_q, c1 = c0 + int64_t(n_kq - n_vq) * c.key_q;
  int64_t t;
  if (target < c0) t = target / c.both_q;
  else if (target < c1) t = n_vq + (target - c0) / c.key_q;
  else t = n_kq + (target - c1) / c.both_16;
  const int64_t ta = t & ~int64_t(kWaveAlign - 1);
  return int(ta < N ? ta : N);
}

hipError_t launch_decode(const DecodeParams& p, int GQ, hipStream_t s);
hipError_t launch_decode_paged(const DecodeParams& p, int GQ, hipStream_t s);
// LDS bytes of a decode workgroup of `waves` waves; -1 if (D, GQ) is unsupported
int64_t decode_lds_bytes(int D, int GQ, int waves);

struct QuantParams {
  const uint16_t* src;
  const int32_t* src_rows;
  uint8_t* codes;
  uint8_t* meta;
  int64_t src_stream_stride, src_row_stride;    // fp16 elements
  int64_t codes_stream_stride, meta_stream_stride;  // bytes
  int32_t bits, G, D, n_streams, n_tok, dst_tok;
};


hipError_t launch_quantize_keys(const QuantParams& p, hipStream_t s);
hipError_t launch_quantize_values(const QuantParams& p, hipStream_t s);
hipError_t launch_decode_append(const AppendParams& p, hipStream_t s);

// fp16 row copy: dst row (dst_row0 + i) of stream s at byte
// s*dst_stream_bytes + (dst_row0+i)*D*2, source row (rows ? rows[i] : i).
hipError_t launch_copy_rows(const uint16_t* src, int64_t src_stream_stride,
                            int64_t src_row_stride, const int32_t* rows,
                            uint8_t* dst, int64_t dst_stream_bytes, int32_t dst_row0,
                            int32_t n_streams, int32_t D, int32_t n_rows, hipStream_t s);

// WindowQuant window-level search (search.hip).
struct SearchParams {
  const uint16_t* text;      // fp16 [B][N][D] rows (strides in elements)
  const uint16_t* visual;    // fp16 [B][M][D]
  int64_t text_batch_stride, text_row_stride, visual_batch_stride, visual_row_stride;
  float* ws;                 // [B][n_chunks][D] chunk sums of unit rows
  float* scores;             // NULL or [B][n_windows]
  uint8_t* win_bits;         // [n_windows]
  int32_t B, N, D, S, n_windows, chunks_per_window, n_chunks, first_window_fp16;
  float t_low, t_high;
};
int32_t search_chunks_per_window(int32_t S);
int64_t search_chunks(int32_t n_text, int32_t n_windows, int32_t S);
hipError_t launch_search(const SearchParams& p, hipStream_t s);

hipError_t launch_reorder(const uint8_t* win_bits, int32_t n_windows, int32_t S,
                          int32_t G, int32_t D, int32_t* perm, void* segs,
                          int32_t* n_segs, int32_t* row_gather, hipStream_t s);

}  // namespace kvq
