// WindowQuant window reorder (ACM TACO, Sec. 3.3.1-3.3.2): windows with the
// same bit width are made contiguous, widest first, keeping the original
// order inside a width (a stable counting sort), and the run table of the
// reordered cache is emitted.
//
// One workgroup of 1024 threads.  Windows are taken 1024 at a time; a block
// scan over a 64-bit word holding four 16-bit per-width counters gives every
// window its rank among the earlier windows of its width in one pass.  The
// row gather list (W * S entries) is written by a second, grid-wide kernel
// from the permutation.

#include <algorithm>

#include "kvq_internal.h"
#include "../../include/kvq.h"

namespace kvq {
namespace {

constexpr int kReorderThreads = 1024;

__device__ __forceinline__ int width_class(uint32_t bits) {
  return bits == 16 ? 0 : bits == 8 ? 1 : bits == 4 ? 2 : bits == 2 ? 3 : -1;
}

__global__ void __launch_bounds__(kReorderThreads) reorder_kernel(
    const uint8_t* win_bits, int32_t W, int32_t S, int32_t G, int32_t D,
    int32_t* perm, kvq_segment* segs, int32_t* n_segs) {
  __shared__ uint64_t scan[kReorderThreads];
  __shared__ int count[4];
  __shared__ int bad;
  const int tid = threadIdx.x;
  if (tid < 4) count[tid] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
  for (int i = tid; i < W; i += kReorderThreads) {
    const int c = width_class(win_bits[i]);
    if (c < 0) atomicOr(&bad, 1);
    else atomicAdd(&count[c], 1);
  }
  __syncthreads();
  if (bad) {
    if (tid == 0) *n_segs = -1;
    return;
  }
  int start[4];
  start[0] = 0;
  for (int c = 1; c < 4; ++c) start[c] = start[c - 1] + count[c - 1];
  uint64_t before = 0;   // windows of each width in earlier chunks, 16-bit fields
  for (int base = 0; base < W; base += kReorderThreads) {
    const int i = base + tid;
    const int c = i < W ? width_class(win_bits[i]) : -1;
    const uint64_t mine = c >= 0 ? (uint64_t(1) << (16 * c)) : 0;
    scan[tid] = mine;
    __syncthreads();
    for (int off = 1; off < kReorderThreads; off <<= 1) {   // inclusive scan
      const uint64_t add = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    if (c >= 0) {
      const uint64_t excl = scan[tid] - mine;
      const int rank = int((excl >> (16 * c)) & 0xffff) + int((before >> (16 * c)) & 0xffff);
      const int pos = start[c] + rank;
      perm[pos] = i;
    }
    // per-width totals of this chunk; a window count fits 16 bits per chunk
    uint64_t total = scan[kReorderThreads - 1];
    __syncthreads();
    for (int c2 = 0; c2 < 4; ++c2) {
      const uint64_t add = (total >> (16 * c2)) & 0xffff;
      const uint64_t cur = (before >> (16 * c2)) & 0xffff;
      before = (before & ~(uint64_t(0xffff) << (16 * c2))) | (((cur + add) & 0xffff) << (16 * c2));
    }
  }
  if (tid == 0) {
    const int widths[4] = {16, 8, 4, 2};
    int n = 0, tok = 0;
    int64_t coff = 0, moff = 0;
    for (int c = 0; c < 4; ++c) {
      if (count[c] == 0) continue;
      const int b = widths[c];
      const int nt = count[c] * S;
      kvq_segment sg;
      sg.bits = b;
      sg.tok_begin = tok;
      sg.n_tok = nt;
      sg.reserved = 0;
      sg.code_off = coff;
      sg.meta_off = moff;
      segs[n++] = sg;
      tok += nt;
      const int64_t cb = b == 16 ? int64_t(nt) * D * 2 : int64_t(nt) * D * b / 8;
      const int64_t mb = b == 16 ? 0 : int64_t(nt) * (D / G) * 4;
      coff = (coff + cb + 255) / 256 * 256;
      moff = (moff + mb + 255) / 256 * 256;
    }
    *n_segs = n;
  }
}

// row_gather[p * S + k] = perm[p] * S + k: entry j of the reordered cache
// reads source row j of window perm[j / S]; nothing when the widths were
// rejected (n_segs < 0, the permutation incomplete).
__global__ void __launch_bounds__(256) row_gather_kernel(const int32_t* perm, const int32_t* n_segs, int32_t S,
                                                         int64_t total, int32_t* row_gather) {
  if (*n_segs < 0) return;
  for (int64_t j = int64_t(blockIdx.x) * 256 + threadIdx.x; j < total; j += int64_t(gridDim.x) * 256)
    row_gather[j] = perm[j / S] * S + int32_t(j % S);
}

}  // namespace

hipError_t launch_reorder(const uint8_t* win_bits, int32_t n_windows, int32_t S,
                          int32_t G, int32_t D, int32_t* perm, void* segs,
                          int32_t* n_segs, int32_t* row_gather, hipStream_t s) {
  hipLaunchKernelGGL(reorder_kernel, dim3(1), dim3(kReorderThreads), 0, s, win_bits,
                     n_windows, S, G, D, perm, static_cast<kvq_segment*>(segs), n_segs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !row_gather) return e;
  const int64_t total = int64_t(n_windows) * S;
  const unsigned grid = unsigned(std::min<int64_t>((total + 255) / 256, 8192));
  hipLaunchKernelGGL(row_gather_kernel, dim3(grid), dim3(256), 0, s, perm, n_segs, S, total, row_gather);
  return hipGetLastError();
}

}  // namespace kvq
