// Internal declarations shared by the host entry points (api.hip) and the
// kernel launchers (quantize.hip, reorder.hip, decode.hip).  Not part of the
// ABI: the ABI is include/kvq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kThreads = 256;          // threads per decode / quantize workgroup
constexpr int kMaxRuns = 8;            // runs per half of the cache
constexpr int kMaxCells = 20;          // token ranges with one key and one value source
constexpr int kRedFloats = kThreads * 32;  // value-reduction buffer (floats)
constexpr int kLdsLimit = 64 * 1024;   // dynamic LDS budget per decode workgroup

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
  int32_t n_kq, n_vq;                   // tokens held in key runs / value runs
  int32_t n_splits, split_tokens;
  float scale_log2;                     // sm_scale * log2(e)
  int32_t n_cells, n_k_runs, n_v_runs;
  Run k_runs[kMaxRuns];
  Run v_runs[kMaxRuns];
  Cell cells[kMaxCells];
};

// Dynamic LDS bytes of one decode workgroup (same carve-up on the device).
inline int64_t decode_lds_bytes(int D, int GQ, int split_tokens, int G) {
  const int64_t ngmax = (split_tokens + G - 1) / G + 1;
  int64_t bytes = 0;
  bytes += int64_t(GQ) * D * 4;            // q * scale, fp32
  bytes += int64_t(GQ) * D * 2;            // q, fp16 pairs
  bytes += ngmax * GQ * D * 2;             // q*s per key group, fp16 pairs
  bytes += ngmax * GQ * 4;                 // bias per key group
  bytes += int64_t(GQ) * split_tokens * 4; // logits / probabilities
  bytes += int64_t(kRedFloats) * 4;        // value reduction
  bytes += 64 * 4;                         // block-reduction scratch
  return bytes;
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
