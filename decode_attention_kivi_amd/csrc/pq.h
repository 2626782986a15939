// Internal declarations of the PQCache decode-time PQ search (pq.hip):
// parameters and launchers shared by pq.hip and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

struct PqParams {
  const uint16_t* q;          // fp16 [B][Hq][D]
  const uint16_t* centroids;  // fp16 [B*Hkv][m][2^bits][D/m]
  const uint8_t* codes;       // u8, stream s at codes + s*codes_stride: [n_tok][m]
  float* scores;              // fp32 [B][Hq][n_tok]
  int32_t* top_idx;           // int32 [B][Hq][top_k]
  int64_t codes_stride;       // bytes
  int32_t B, Hq, Hkv, gq, D, m, bits, n_tok, top_k, chunk_tokens;
};
// LDS of the scores kernel (the tables of a kv head's GQ query heads)
int64_t pq_scores_lds_bytes(int gq_pow2, int D, int m, int bits);
// LDS of the one-kernel search (a head's scores resident in LDS)
int64_t pq_fused_lds_bytes(int n_tok, int D, int m, int bits);
// fused: one workgroup per query head with its scores in LDS (the LDS must
// hold pq_fused_lds_bytes); else the scores kernel, then the Top-k kernel
hipError_t launch_pq_search(const PqParams& p, int GQ, bool fused, hipStream_t s);

}  // namespace kvq
