// Internal declarations of decode attention over a vector-quantized
// (codebook) KV cache (vq.hip): parameters and launchers shared by vq.hip
// and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

struct VqParams {
  const uint16_t* q;          // fp16 [B][Hq][D]
  const uint8_t* k_codes;     // u8, stream s at k_codes + s*codes_stride: [n_tok][R][D/4]
  const uint8_t* v_codes;     // likewise
  const uint16_t* k_books;    // fp16 [Hkv][R][D/4][256][4]
  const uint16_t* v_books;    // likewise
  float* out;                 // fp32 [B][Hq][D]
  float* ws;                  // partial states [stream][chunk][gq][D + 2] when n_chunks > 1
  int64_t codes_stride;       // bytes
  int32_t B, Hq, Hkv, gq, D, R, n_tok, chunk_tokens, n_chunks;
  float scale_log2;           // sm_scale * log2(e)
};

constexpr int kVqMaxChunk = 8192;       // tokens per workgroup at most
constexpr int kVqMaxChunks = 1024;      // chunks per stream at most

// LDS region of the partial kernel, one codebook round at a time: a round's
// key table (D/4 * 256 fp32) and the chunk's logits (fp32) first, the
// round's value codebook (D/4 * 256 * 4 fp16) after them
__host__ __device__ inline int64_t vq_region_bytes(int D, int chunk_tokens) {
  const int64_t ne = int64_t(D / 4) * 256;
  const int64_t a = ne * 8, b = (ne + chunk_tokens) * 4;
  return ((a > b ? a : b) + 15) / 16 * 16;
}
// LDS bytes of the partial kernel (region, fp16 probabilities, q)
int64_t vq_lds_bytes(int D, int chunk_tokens);
hipError_t launch_vq_decode(const VqParams& p, hipStream_t s);

}  // namespace kvq
