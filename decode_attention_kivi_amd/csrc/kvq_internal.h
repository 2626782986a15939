// Internal declarations shared by the host entry points (api.hip) and the
// kernel launchers (quantize.hip, reorder.hip, decode.hip).  Not part of the
// ABI: the ABI is include/kvq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kThreads = 256;          // threads per decode / quantize workgroup
constexpr int kWaves = 4;              // waves per decode workgroup
constexpr int kMaxRuns = 8;            // runs per half of the cache
constexpr int kMaxCells = 20;          // token ranges with one key and one value source
constexpr int kLdsLimit = 64 * 1024;   // dynamic LDS budget per decode workgroup

// Tokens each wave of a decode workgroup streams; a workgroup covers
// kWaves * wave_tokens(GQ) tokens.  Larger GQ needs more LDS per token.
__host__ __device__ constexpr int wave_tokens(int GQ) { return GQ <= 1 ? 256 : GQ == 2 ? 128 : GQ == 4 ? 64 : 32; }

struct Run {            // device copy of kvq_segment
  int32_t bits, tok_begin, n_tok, pad;
  int64_t code_off, meta_off;
};

// A maximal token range [t0, t0+n) whose keys come from one source and whose
// values come from one source.  k_src / v_src: run index, or -1 = residual.
struct Cell {
  int32_t t0, n, k_src, v_src, split0, pad0, pad1, pad2;
};

struct DecodeParams {
  const uint16_t* q;
  float* out;
  float* ws;
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
  int32_t n_kq, n_vq;                   // tokens held in key runs / value runs
  int32_t n_splits, split_tokens;       // split_tokens = kWaves * wave_tokens(GQ)
  float scale_log2;                     // sm_scale * log2(e)
  int32_t n_cells, n_k_runs, n_v_runs;
  Run k_runs[kMaxRuns];
  Run v_runs[kMaxRuns];
  Cell cells[kMaxCells];
};

// LDS carve-up of one decode workgroup (the device uses the same numbers).
// Block part: q of the GQ heads as fp16.  Per wave, for LT = wave_tokens + 4
// token slots (a leading slot keeps value pairs aligned, the tail is zero):
//   logit  fp32 [GQ][LT]  logits; reused afterwards for the [4][D] value
//                          reduction rows
//   p16    fp16 [GQ][LT]  probabilities, zero outside the wave's tokens
//   area   q*s hi/lo pairs [NGW][GQ][2][D/2] and bias [NGW][GQ] per key group
//          (NGW groups, sized for G = 32); afterwards the wave's partial
//          (m, l, o[D]) per head
struct DecodeLds {
  int64_t block, logit, p16, area, wave, total;
};
__host__ __device__ constexpr int64_t round16(int64_t x) { return (x + 15) / 16 * 16; }
__host__ __device__ constexpr int64_t cmax(int64_t a, int64_t b) { return a > b ? a : b; }
__host__ __device__ constexpr DecodeLds decode_lds(int D, int GQ) {
  const int64_t lt = wave_tokens(GQ) + 4;
  const int64_t ngw = wave_tokens(GQ) / 32 + 1;
  const int64_t block = round16(int64_t(GQ) * D * 2);
  const int64_t logit = round16(cmax(int64_t(GQ) * lt * 4, int64_t(4) * D * 4));
  const int64_t p16 = round16(int64_t(GQ) * lt * 2);
  const int64_t area = round16(cmax(ngw * GQ * D * 4 + ngw * GQ * 4, int64_t(GQ) * (D + 2) * 4));
  const int64_t wave = logit + p16 + area;
  return DecodeLds{block, logit, p16, area, wave, block + kWaves * wave};
}

hipError_t launch_decode(const DecodeParams& p, int GQ, hipStream_t s);

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

// fp16 row copy: dst row (dst_row0 + i) of stream s at byte
// s*dst_stream_bytes + (dst_row0+i)*D*2, source row (rows ? rows[i] : i).
hipError_t launch_copy_rows(const uint16_t* src, int64_t src_stream_stride,
                            int64_t src_row_stride, const int32_t* rows,
                            uint8_t* dst, int64_t dst_stream_bytes, int32_t dst_row0,
                            int32_t n_streams, int32_t D, int32_t n_rows, hipStream_t s);

hipError_t launch_reorder(const uint8_t* win_bits, int32_t n_windows, int32_t S,
                          int32_t G, int32_t D, int32_t* perm, void* segs,
                          int32_t* n_segs, int32_t* row_gather, hipStream_t s);

}  // namespace kvq
