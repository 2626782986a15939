// extern "C" entry points of include/kvq.h: argument checks on the host,
// launch planning, kernel launches.  No allocation, no synchronization.

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/kvq.h"
#include "kvq_internal.h"
#include "pq.h"
#include "vq.h"

namespace {

using kvq::DecodeParams;
using kvq::Run;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool valid_d(int d) { return d == 64 || d == 128; }
bool valid_group(int g) { return g == 32 || g == 64 || g == 128; }
bool valid_bits(int b) { return b == 2 || b == 4 || b == 8 || b == 16; }

kvq_status from_hip(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ELAUNCH; }

// The launch plan of one decode call, derived from the arguments alone.
struct Plan {
  DecodeParams p;
  int GQ = 1;
  size_t ws_bytes = 0;
};

kvq_status check_runs(const kvq_segment* segs, int n, int d, int G, bool keys, int64_t* n_total) {
  if (n < 0 || n > kvq::kMaxRuns) return KVQ_EINVAL;
  if (n > 0 && !segs) return KVQ_EINVAL;
  int64_t tok = 0;
  for (int i = 0; i < n; ++i) {
    const kvq_segment& s = segs[i];
    if (!valid_bits(s.bits) || s.reserved != 0) return KVQ_EINVAL;
    if (s.n_tok < 0 || s.tok_begin != tok) return KVQ_EINVAL;
    if (s.code_off < 0 || s.meta_off < 0) return KVQ_EINVAL;
    if ((s.code_off & 15) || (s.meta_off & 15)) return KVQ_EALIGN;
    if (keys && s.bits != 16 && s.n_tok % G != 0) return KVQ_EINVAL;
    // quantized key runs start on a group boundary, quantized value runs on
    // a pair boundary (true of every run the library's own calls produce)
    if (keys && s.bits != 16 && s.tok_begin % G != 0) return KVQ_EUNSUPPORTED;
    if (!keys && s.bits != 16 && (s.tok_begin & 1)) return KVQ_EUNSUPPORTED;
    (void)d;
    tok += s.n_tok;
  }
  *n_total = tok;
  return KVQ_OK;
}

kvq_status make_plan(const kvq_decode_args* a, Plan* out) {
  if (!a) return KVQ_EINVAL;
  if (a->batch < 1 || a->n_kv_heads < 1 || a->n_q_heads < 1) return KVQ_EINVAL;
  if (a->n_q_heads % a->n_kv_heads != 0) return KVQ_EINVAL;
  const int gq = a->n_q_heads / a->n_kv_heads;
  if (!valid_d(a->d_h) || !valid_group(a->group) || a->group > a->d_h) return KVQ_EUNSUPPORTED;
  if (int64_t(a->batch) * a->n_kv_heads > 65535) return KVQ_EUNSUPPORTED;
  if (!(std::isfinite(a->sm_scale))) return KVQ_EINVAL;
  if (!a->q || !a->out) return KVQ_EINVAL;
  if (a->n_k_res < 0 || a->n_v_res < 0 || a->split_tokens < 0) return KVQ_EINVAL;
  const int D = a->d_h, G = a->group;

  int64_t nk = 0, nv = 0;
  kvq_status st = check_runs(a->k_segs, a->n_k_segs, D, G, true, &nk);
  if (st != KVQ_OK) return st;
  st = check_runs(a->v_segs, a->n_v_segs, D, G, false, &nv);
  if (st != KVQ_OK) return st;
  const int64_t N = nk + a->n_k_res;
  if (N < 1 || N != nv + a->n_v_res || N > (int64_t(1) << 30)) return KVQ_EINVAL;
  bool k_quant = false, v_quant = false;
  for (int i = 0; i < a->n_k_segs; ++i) k_quant |= a->k_segs[i].bits != 16 && a->k_segs[i].n_tok > 0;
  for (int i = 0; i < a->n_v_segs; ++i) v_quant |= a->v_segs[i].bits != 16 && a->v_segs[i].n_tok > 0;
  if ((nk > 0 && !a->k_codes) || (k_quant && !a->k_meta)) return KVQ_EINVAL;
  if ((nv > 0 && !a->v_codes) || (v_quant && !a->v_meta)) return KVQ_EINVAL;
  if (a->n_k_res > 0 && !a->k_res) return KVQ_EINVAL;
  if (a->n_v_res > 0 && !a->v_res) return KVQ_EINVAL;
  for (const void* ptr : {a->q, static_cast<const void*>(a->out), a->k_codes, a->k_meta,
                          a->v_codes, a->v_meta, a->k_res, a->v_res, static_cast<const void*>(a->workspace)})
    if (ptr && !aligned16(ptr)) return KVQ_EALIGN;
  for (int64_t s : {a->k_codes_stride, a->k_meta_stride, a->v_codes_stride, a->v_meta_stride})
    if (s < 0 || (s & 15)) return s < 0 ? KVQ_EINVAL : KVQ_EALIGN;
  for (int64_t s : {a->k_res_stride, a->v_res_stride})
    if (s < 0 || (s & 7)) return s < 0 ? KVQ_EINVAL : KVQ_EALIGN;

  // head blocks of up to 4 query heads per workgroup (grid z)
  const int GQ = kvq::decode_head_block(gq);
  const int64_t hblocks = (gq + GQ - 1) / GQ;
  if (kvq::decode_lds_bytes(D, GQ, 4) < 0) return KVQ_EUNSUPPORTED;
  const int64_t streams = int64_t(a->batch) * a->n_kv_heads;
  // Cost pieces: maximal token ranges with one key source and one value
  // source, priced in HBM bytes per token.
  std::vector<kvq::CostPiece> pieces;
  {
    std::vector<int64_t> cuts = {0, N, nk, nv};
    for (int i = 0; i < a->n_k_segs; ++i) cuts.push_back(a->k_segs[i].tok_begin);
    for (int i = 0; i < a->n_v_segs; ++i) cuts.push_back(a->v_segs[i].tok_begin);
    std::sort(cuts.begin(), cuts.end());
    cuts.erase(std::unique(cuts.begin(), cuts.end()), cuts.end());
    auto row_cost = [&](int bits, bool keys) -> int64_t {
      if (bits == 16) return int64_t(D) * 2;
      return int64_t(D) * bits / 8 + (keys ? int64_t(D) * 4 / G : int64_t(D / G) * 4);
    };
    int64_t c = 0;
    for (size_t i = 0; i + 1 < cuts.size(); ++i) {
      const int64_t t0 = cuts[i], t1 = cuts[i + 1];
      if (t1 <= t0) continue;
      int kb = 16, vb = 16;
      for (int k = 0; k < a->n_k_segs; ++k)
        if (t0 >= a->k_segs[k].tok_begin && t0 < a->k_segs[k].tok_begin + a->k_segs[k].n_tok) kb = a->k_segs[k].bits;
      for (int k = 0; k < a->n_v_segs; ++k)
        if (t0 >= a->v_segs[k].tok_begin && t0 < a->v_segs[k].tok_begin + a->v_segs[k].n_tok) vb = a->v_segs[k].bits;
      const int64_t cost = row_cost(kb, true) + row_cost(vb, false);
      pieces.push_back(kvq::CostPiece{int32_t(t0), int32_t(cost), c});
      c += (t1 - t0) * cost;
    }
    if (pieces.empty() || pieces.size() > size_t(kvq::kMaxPieces)) return KVQ_EUNSUPPORTED;
  }
  const int64_t cost_total = pieces.back().c0 + (N - pieces.back().t0) * pieces.back().cost;

  // Each stream's N tokens are cut into nw * n_wg wave ranges of about
  // equal cost, nw = decode_waves(D, GQ) waves per workgroup.  The automatic
  // choice takes the n_wg with the least (rounds of the grid over the chip)
  // x (tokens per workgroup), ties to fewer workgroups (n_wg = 1: no partial
  // states, no merge kernel), among the counts whose waves hold at least 64
  // tokens and at most wave_cap(GQ); split_tokens > 0 asks for workgroups of
  // that many tokens (refused when a wave range would exceed wave_cap(GQ)).
  auto longest = [&](int64_t nws) {
    int64_t worst = 0;
    int prev = 0;
    for (int64_t w = 1; w <= nws; ++w) {
      const int b = kvq::wave_bound(pieces.data(), int(pieces.size()), cost_total, int(N), int(w), int(nws));
      worst = std::max<int64_t>(worst, b - prev);
      prev = b;
    }
    return worst;
  };
  int nw = kvq::decode_waves(D, GQ);
  int64_t n_wg;
  if (a->split_tokens > 0) {
    n_wg = (N + a->split_tokens - 1) / a->split_tokens;
    if (n_wg > (int64_t(1) << 20)) return KVQ_EUNSUPPORTED;
    if (longest(nw * n_wg) > kvq::wave_cap(GQ)) return KVQ_EUNSUPPORTED;
  } else {
    const int64_t fill = 256 * kvq::decode_wgs_per_cu(GQ);   // workgroups resident at once
    int64_t n_min = std::max<int64_t>(1, (N + int64_t(nw) * kvq::wave_tokens(GQ) * 3 / 2 - 1) /
                                             (int64_t(nw) * kvq::wave_tokens(GQ) * 3 / 2));
    while (longest(nw * n_min) > kvq::wave_cap(GQ)) {
      if (n_min >= (int64_t(1) << 20)) return KVQ_EUNSUPPORTED;
      n_min += std::max<int64_t>(1, n_min / 8);
    }
    n_wg = n_min;
    double best = -1;
    for (int64_t c = n_min; c <= std::min(8 * n_min, n_min + 256); ++c) {
      if (c > n_min && (N + nw * c - 1) / (nw * c) < 64) break;
      const double rounds = double((streams * hblocks * c + fill - 1) / fill);
      const double t = rounds * double(N) / double(c);
      if (best >= 0 && t >= best * (1 - 1e-9)) continue;
      // the wave-length check walks every wave bound: only for a candidate
      // that would be taken
      if (c > n_min && longest(nw * c) > kvq::wave_cap(GQ)) continue;
      best = t;
      n_wg = c;
    }
    // One head per kv head, more streams than the chip holds at once, each
    // in one workgroup: 4-wave workgroups (four per CU instead of two 8-wave
    // ones) give each wave twice the tokens at the same occupancy, so the
    // per-wave fixed costs (prologue, load ramps, softmax, combine) are paid
    // half as often (batch-64 int2, 2049 tokens: 86.5 -> 77.9 us); with the
    // chip filled once they would only split streams across workgroups.
    if (GQ == 1 && D == 128 && n_wg == 1 && streams * hblocks > fill &&
        longest(kvq::kWavesSmall) <= kvq::wave_cap(GQ))
      nw = kvq::kWavesSmall;
  }
  const int64_t nws = nw * n_wg;
  if (kvq::decode_lds_bytes(D, GQ, nw) > kvq::kLdsLimit) return KVQ_EUNSUPPORTED;

  Plan& pl = *out;
  DecodeParams& p = pl.p;
  std::memset(&p, 0, sizeof(p));
  p.q = static_cast<const uint16_t*>(a->q);
  p.out = a->out;
  p.ws = static_cast<float*>(a->workspace);
  p.k_codes = static_cast<const uint8_t*>(a->k_codes);
  p.k_meta = static_cast<const uint8_t*>(a->k_meta);
  p.v_codes = static_cast<const uint8_t*>(a->v_codes);
  p.v_meta = static_cast<const uint8_t*>(a->v_meta);
  p.k_res = static_cast<const uint16_t*>(a->k_res);
  p.v_res = static_cast<const uint16_t*>(a->v_res);
  p.k_codes_stride = a->k_codes_stride;
  p.k_meta_stride = a->k_meta_stride;
  p.v_codes_stride = a->v_codes_stride;
  p.v_meta_stride = a->v_meta_stride;
  p.k_res_stride = a->k_res_stride;
  p.v_res_stride = a->v_res_stride;
  p.B = a->batch;
  p.Hq = a->n_q_heads;
  p.Hkv = a->n_kv_heads;
  p.D = D;
  p.G = G;
  p.lg_g = G == 32 ? 5 : G == 64 ? 6 : 7;
  p.gq = gq;
  p.n_tok = int32_t(N);
  p.n_kq = int32_t(nk);
  p.n_vq = int32_t(nv);
  p.waves_per_stream = int32_t(nws);
  p.waves_per_wg = nw;
  p.wg_per_stream = int32_t(n_wg);
  p.scale_log2 = a->sm_scale * 1.4426950408889634f;
  p.n_pieces = int32_t(pieces.size());
  p.cost_total = cost_total;
  for (size_t i = 0; i < pieces.size(); ++i) p.pieces[i] = pieces[i];
  if (nws <= kvq::kMaxBounds) {
    p.n_bounds = int32_t(nws + 1);
    for (int64_t w = 0; w <= nws; ++w)
      p.bounds[w] = kvq::wave_bound(pieces.data(), int(pieces.size()), cost_total, int(N), int(w), int(nws));
  }
  p.n_k_runs = a->n_k_segs;
  p.n_v_runs = a->n_v_segs;
  for (int i = 0; i < a->n_k_segs; ++i)
    p.k_runs[i] = Run{a->k_segs[i].bits, a->k_segs[i].tok_begin, a->k_segs[i].n_tok, 0,
                      a->k_segs[i].code_off, a->k_segs[i].meta_off};
  for (int i = 0; i < a->n_v_segs; ++i)
    p.v_runs[i] = Run{a->v_segs[i].bits, a->v_segs[i].tok_begin, a->v_segs[i].n_tok, 0,
                      a->v_segs[i].code_off, a->v_segs[i].meta_off};
  pl.GQ = GQ;
  // the per-workgroup partial states; one workgroup per stream writes the
  // output directly and needs no workspace
  pl.ws_bytes = n_wg == 1 ? 0
                          : size_t(streams) * size_t(n_wg) * size_t(gq) * size_t(D + 2) * sizeof(float);
  return KVQ_OK;
}

// Page layout (kvq_page_layout): a key run and a value run of PT tokens per
// kv head, head blocks back to back.
struct PageLayout {
  int64_t head_bytes, kmeta_off, vcodes_off, vmeta_off, page_bytes;
};
kvq_status page_layout(int n_kv_heads, int d_h, int group, int bits, int page_tokens, PageLayout* out) {
  if (n_kv_heads < 1 || page_tokens < 1) return KVQ_EINVAL;
  if (bits != 2 && bits != 4 && bits != 8) return KVQ_EINVAL;
  if (!valid_d(d_h) || !valid_group(group) || group > d_h) return KVQ_EUNSUPPORTED;
  if (page_tokens % 64 != 0 || page_tokens % group != 0 || page_tokens > 65536) return KVQ_EUNSUPPORTED;
  const int64_t PT = page_tokens, rb = int64_t(d_h) * bits / 8;
  PageLayout L;
  L.kmeta_off = PT * rb;
  L.vcodes_off = L.kmeta_off + PT / group * d_h * 4;
  L.vmeta_off = L.vcodes_off + PT * rb;
  L.head_bytes = kvq::round16(L.vmeta_off + PT * (d_h / group) * 4);
  L.page_bytes = L.head_bytes * n_kv_heads;
  *out = L;
  return KVQ_OK;
}

kvq_status make_paged_plan(const kvq_paged_args* a, Plan* out) {
  if (!a) return KVQ_EINVAL;
  if (a->batch < 1 || a->n_kv_heads < 1 || a->n_q_heads < 1) return KVQ_EINVAL;
  if (a->n_q_heads % a->n_kv_heads != 0) return KVQ_EINVAL;
  const int gq = a->n_q_heads / a->n_kv_heads;
  if (int64_t(a->batch) * a->n_kv_heads > 65535) return KVQ_EUNSUPPORTED;
  PageLayout L;
  kvq_status st = page_layout(a->n_kv_heads, a->d_h, a->group, a->bits, a->page_tokens, &L);
  if (st != KVQ_OK) return st;
  if (!std::isfinite(a->sm_scale)) return KVQ_EINVAL;
  if (!a->q || !a->out || !a->pages || !a->block_table || !a->lengths || !a->lengths_dev) return KVQ_EINVAL;
  if (a->max_pages < 1 || a->page_bytes < L.page_bytes) return KVQ_EINVAL;
  if (a->page_bytes & 15) return KVQ_EALIGN;
  for (const void* ptr : {a->q, static_cast<const void*>(a->out), a->pages, a->k_res, a->v_res,
                          static_cast<const void*>(a->workspace)})
    if (ptr && !aligned16(ptr)) return KVQ_EALIGN;
  if ((reinterpret_cast<uintptr_t>(a->block_table) & 3) || (reinterpret_cast<uintptr_t>(a->lengths_dev) & 3))
    return KVQ_EALIGN;
  for (int64_t s : {a->k_res_stride, a->v_res_stride})
    if (s < 0 || (s & 7)) return s < 0 ? KVQ_EINVAL : KVQ_EALIGN;
  const int D = a->d_h, G = a->group;
  const int GQ = kvq::decode_head_block(gq);     // head blocks of up to 4 query heads (grid z)
  const int nw = GQ == 1 && D == 128 ? kvq::kWavesSmall : kvq::decode_waves(D, GQ);
  if (kvq::decode_lds_bytes(D, GQ, nw) > kvq::kLdsLimit) return KVQ_EUNSUPPORTED;
  const kvq::PagedCost pc = kvq::paged_cost(D, G, a->bits);
  // workgroups per stream: waves of up to wave_cap(GQ) - kWaveAlign tokens
  // of the cheapest kind (the longest ranges the LDS slots hold: fewer
  // workgroups and wave restarts; 78.4 against 79.6-80.9 us at 512 tokens
  // on the ragged bench batch, 88.7 at 256, 109 at 128)
  const int wt = kvq::wave_cap(GQ) - kvq::kWaveAlign;
  int wg_max = 1;
  bool any_kres = false, any_vres = false;
  std::vector<std::pair<double, int>> order;      // (-cost per workgroup, sequence)
  std::vector<int> seq_wgs(a->batch);
  for (int b = 0; b < a->batch; ++b) {
    const int64_t nk = a->lengths[4 * b], nv = a->lengths[4 * b + 1];
    const int64_t rk = a->lengths[4 * b + 2], rv = a->lengths[4 * b + 3];
    if (nk < 0 || nv < 0 || rk < 0 || rv < 0 || nv > nk || nk % G != 0) return KVQ_EINVAL;
    const int64_t N = nk + rk;
    if (N != nv + rv || N < 1 || N > (int64_t(1) << 22)) return KVQ_EINVAL;
    if ((nk + a->page_tokens - 1) / a->page_tokens > a->max_pages) return KVQ_EINVAL;
    any_kres |= rk > 0;
    any_vres |= rv > 0;
    const int nwg = kvq::paged_wgs(pc, int(nk), int(nv), int(N), wt, nw);
    wg_max = std::max(wg_max, nwg);
    seq_wgs[b] = nwg;
    order.emplace_back(-double(kvq::paged_total(pc, int(nk), int(nv), int(N))) / nwg, b);
  }
  if ((any_kres && !a->k_res) || (any_vres && !a->v_res)) return KVQ_EINVAL;
  if (wg_max > (1 << 16)) return KVQ_EUNSUPPORTED;

  Plan& pl = *out;
  DecodeParams& p = pl.p;
  std::memset(&p, 0, sizeof(p));
  p.q = static_cast<const uint16_t*>(a->q);
  p.out = a->out;
  p.ws = static_cast<float*>(a->workspace);
  p.k_res = static_cast<const uint16_t*>(a->k_res);
  p.v_res = static_cast<const uint16_t*>(a->v_res);
  p.k_res_stride = a->k_res_stride;
  p.v_res_stride = a->v_res_stride;
  p.B = a->batch;
  p.Hq = a->n_q_heads;
  p.Hkv = a->n_kv_heads;
  p.D = D;
  p.G = G;
  p.lg_g = G == 32 ? 5 : G == 64 ? 6 : 7;
  p.gq = gq;
  p.waves_per_wg = nw;
  p.wg_per_stream = wg_max;
  p.scale_log2 = a->sm_scale * 1.4426950408889634f;
  p.pages = static_cast<const uint8_t*>(a->pages);
  p.block_table = a->block_table;
  p.lens = a->lengths_dev;
  p.page_bytes = a->page_bytes;
  p.head_bytes = L.head_bytes;
  p.page_tokens = a->page_tokens;
  p.max_pages = a->max_pages;
  p.pg_kmeta_off = int32_t(L.kmeta_off);
  p.pg_vcodes_off = int32_t(L.vcodes_off);
  p.pg_vmeta_off = int32_t(L.vmeta_off);
  p.bits = a->bits;
  p.pg_wave_tokens = wt;
  if (a->batch <= kvq::kMaxSched) {
    // heaviest workgroups first (longest-processing-time order), so the
    // longest sequences do not start last; stable for equal costs
    std::stable_sort(order.begin(), order.end(),
                     [](const std::pair<double, int>& x, const std::pair<double, int>& y) { return x.first < y.first; });
    int64_t acc = 0;
    p.sched_n = a->batch;
    for (int k = 0; k < a->batch; ++k) {
      const int b = order[k].second;
      p.sched_seq[k] = uint16_t(b);
      p.sched_start[k] = int32_t(acc);
      acc += int64_t(seq_wgs[b]) * a->n_kv_heads;
    }
    if (acc > INT32_MAX) return KVQ_EUNSUPPORTED;
    p.sched_start[a->batch] = int32_t(acc);
  }
  pl.GQ = GQ;
  pl.ws_bytes = wg_max == 1 ? 0
                            : size_t(a->batch) * size_t(a->n_kv_heads) * size_t(wg_max) * size_t(gq) *
                                  size_t(D + 2) * sizeof(float);
  return KVQ_OK;
}

}  // namespace

extern "C" {

int32_t kvq_abi_version(void) { return KVQ_ABI_VERSION; }

const char* kvq_strerror(int32_t status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_EINVAL: return "invalid argument";
    case KVQ_EALIGN: return "misaligned pointer, offset or stride";
    case KVQ_EUNSUPPORTED: return "unsupported shape";
    case KVQ_EWORKSPACE: return "workspace missing or too small";
    case KVQ_ELAUNCH: return "kernel launch failed";
    case KVQ_ESCRATCH: return "partial states exceed the library's static scratch (KVQ_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

kvq_status kvq_quantize_append(int32_t which, int32_t bits, int32_t group, int32_t n_streams,
                               int32_t d_h, int32_t n_tok, const void* src,
                               int64_t src_stream_stride, int64_t src_row_stride,
                               const int32_t* src_rows, void* codes,
                               int64_t codes_stream_stride, void* meta,
                               int64_t meta_stream_stride, int32_t dst_tok, void* stream) {
  if (which != KVQ_KEYS && which != KVQ_VALUES) return KVQ_EINVAL;
  if (!valid_bits(bits)) return KVQ_EINVAL;
  if (!valid_group(group) || !valid_d(d_h)) return KVQ_EUNSUPPORTED;
  if (which == KVQ_VALUES && bits != 16 && group > d_h) return KVQ_EUNSUPPORTED;
  if (n_streams < 1 || n_tok < 0 || dst_tok < 0) return KVQ_EINVAL;
  if (n_streams > 65535) return KVQ_EUNSUPPORTED;
  if (which == KVQ_KEYS && bits != 16 && (n_tok % group != 0 || dst_tok % group != 0))
    return KVQ_EINVAL;
  if (!src || !codes || (bits != 16 && !meta)) return KVQ_EINVAL;
  if (src_stream_stride < 0 || src_row_stride < d_h || codes_stream_stride < 0 ||
      meta_stream_stride < 0)
    return KVQ_EINVAL;
  if (!aligned16(src) || !aligned16(codes) || (meta && !aligned16(meta))) return KVQ_EALIGN;
  if ((src_stream_stride & 7) || (src_row_stride & 7) || (codes_stream_stride & 15) ||
      (meta_stream_stride & 15))
    return KVQ_EALIGN;
  if (int64_t(dst_tok) + n_tok > (int64_t(1) << 30)) return KVQ_EINVAL;
  if (n_tok == 0) return KVQ_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bits == 16)
    return from_hip(kvq::launch_copy_rows(static_cast<const uint16_t*>(src), src_stream_stride,
                                          src_row_stride, src_rows, static_cast<uint8_t*>(codes),
                                          codes_stream_stride, dst_tok, n_streams, d_h, n_tok, s));
  kvq::QuantParams p{};
  p.src = static_cast<const uint16_t*>(src);
  p.src_rows = src_rows;
  p.codes = static_cast<uint8_t*>(codes);
  p.meta = static_cast<uint8_t*>(meta);
  p.src_stream_stride = src_stream_stride;
  p.src_row_stride = src_row_stride;
  p.codes_stream_stride = codes_stream_stride;
  p.meta_stream_stride = meta_stream_stride;
  p.bits = bits;
  p.G = group;
  p.D = d_h;
  p.n_streams = n_streams;
  p.n_tok = n_tok;
  p.dst_tok = dst_tok;
  return from_hip(which == KVQ_KEYS ? kvq::launch_quantize_keys(p, s)
                                    : kvq::launch_quantize_values(p, s));
}

kvq_status kvq_residual_append(int32_t n_streams, int32_t d_h, int32_t n_rows, const void* src,
                               int64_t src_stream_stride, int64_t src_row_stride, void* dst,
                               int64_t dst_stream_stride, int32_t dst_row, void* stream) {
  if (!valid_d(d_h)) return KVQ_EUNSUPPORTED;
  if (n_streams < 1 || n_rows < 0 || dst_row < 0) return KVQ_EINVAL;
  if (!src || !dst) return KVQ_EINVAL;
  if (src_stream_stride < 0 || src_row_stride < d_h || dst_stream_stride < 0) return KVQ_EINVAL;
  if (!aligned16(src) || !aligned16(dst)) return KVQ_EALIGN;
  if ((src_stream_stride & 7) || (src_row_stride & 7) || (dst_stream_stride & 7)) return KVQ_EALIGN;
  if (n_rows == 0) return KVQ_OK;
  return from_hip(kvq::launch_copy_rows(static_cast<const uint16_t*>(src), src_stream_stride,
                                        src_row_stride, nullptr, static_cast<uint8_t*>(dst),
                                        dst_stream_stride * 2, dst_row, n_streams, d_h, n_rows,
                                        static_cast<hipStream_t>(stream)));
}

kvq_status kvq_decode_append(int32_t bits, int32_t group, int32_t n_streams, int32_t d_h,
                             const void* k_new, int64_t k_new_stride,
                             const void* v_new, int64_t v_new_stride,
                             void* k_res, int64_t k_res_stride, int32_t k_row,
                             void* v_res, int64_t v_res_stride, int32_t v_row,
                             int32_t v_quant_row,
                             void* v_codes, int64_t v_codes_stride,
                             void* v_meta, int64_t v_meta_stride, int32_t v_dst_tok,
                             void* stream) {
  if (bits != 2 && bits != 4 && bits != 8) return KVQ_EINVAL;
  if (!valid_group(group) || !valid_d(d_h) || group > d_h) return KVQ_EUNSUPPORTED;
  if (n_streams < 1 || k_row < 0 || v_row < 0 || v_quant_row < -1) return KVQ_EINVAL;
  if (n_streams > (1 << 24)) return KVQ_EUNSUPPORTED;
  if (!k_new || !v_new || !k_res || !v_res) return KVQ_EINVAL;
  if (k_new_stride < d_h || v_new_stride < d_h || k_res_stride < 0 || v_res_stride < 0)
    return KVQ_EINVAL;
  for (const void* ptr : {k_new, v_new, static_cast<const void*>(k_res), static_cast<const void*>(v_res)})
    if (!aligned16(ptr)) return KVQ_EALIGN;
  if ((k_new_stride & 7) || (v_new_stride & 7) || (k_res_stride & 7) || (v_res_stride & 7))
    return KVQ_EALIGN;
  if (v_quant_row >= 0) {
    if (!v_codes || !v_meta || v_dst_tok < 0 || v_codes_stride < 0 || v_meta_stride < 0)
      return KVQ_EINVAL;
    if (!aligned16(v_codes) || !aligned16(v_meta) || (v_codes_stride & 15) || (v_meta_stride & 15))
      return KVQ_EALIGN;
  }
  kvq::AppendParams p{};
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.k_res = static_cast<uint16_t*>(k_res);
  p.v_res = static_cast<uint16_t*>(v_res);
  p.v_codes = static_cast<uint8_t*>(v_codes);
  p.v_meta = static_cast<uint8_t*>(v_meta);
  p.k_new_stride = k_new_stride;
  p.v_new_stride = v_new_stride;
  p.k_res_stride = k_res_stride;
  p.v_res_stride = v_res_stride;
  p.v_codes_stride = v_codes_stride;
  p.v_meta_stride = v_meta_stride;
  p.bits = bits;
  p.G = group;
  p.D = d_h;
  p.n_streams = n_streams;
  p.k_row = k_row;
  p.v_row = v_row;
  p.v_quant_row = v_quant_row;
  p.v_dst_tok = v_dst_tok;
  return from_hip(kvq::launch_decode_append(p, static_cast<hipStream_t>(stream)));
}

kvq_status kvq_reorder_windows(const uint8_t* win_bits, int32_t n_windows, int32_t window_tokens,
                               int32_t group, int32_t d_h, int32_t* perm, kvq_segment* segs,
                               int32_t* n_segs, int32_t* row_gather, void* stream) {
  if (!valid_group(group) || !valid_d(d_h) || group > d_h) return KVQ_EUNSUPPORTED;
  if (n_windows < 1 || n_windows > 65536) return KVQ_EINVAL;
  if (window_tokens < 1 || window_tokens % group != 0 || (window_tokens & 1)) return KVQ_EINVAL;
  if (int64_t(n_windows) * window_tokens > (int64_t(1) << 30)) return KVQ_EINVAL;
  if (!win_bits || !perm || !segs || !n_segs) return KVQ_EINVAL;
  if ((reinterpret_cast<uintptr_t>(perm) & 3) || (reinterpret_cast<uintptr_t>(n_segs) & 3) ||
      (reinterpret_cast<uintptr_t>(row_gather) & 3) || (reinterpret_cast<uintptr_t>(segs) & 7))
    return KVQ_EALIGN;
  return from_hip(kvq::launch_reorder(win_bits, n_windows, window_tokens, group, d_h, perm, segs,
                                      n_segs, row_gather, static_cast<hipStream_t>(stream)));
}

kvq_status kvq_decode_attn_workspace(const kvq_decode_args* args, size_t* bytes) {
  if (!bytes) return KVQ_EINVAL;
  Plan pl;
  const kvq_status st = make_plan(args, &pl);
  if (st != KVQ_OK) return st;
  *bytes = pl.ws_bytes;
  return KVQ_OK;
}

kvq_status kvq_decode_attn(const kvq_decode_args* args, void* stream) {
  Plan pl;
  const kvq_status st = make_plan(args, &pl);
  if (st != KVQ_OK) return st;
  if (pl.ws_bytes > 0 && (!args->workspace || args->workspace_bytes < pl.ws_bytes))
    return KVQ_EWORKSPACE;
  return from_hip(kvq::launch_decode(pl.p, pl.GQ, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Decode attention for callers that cannot allocate: the partial softmax
// states go to a file-scope device array instead of a caller workspace.
namespace {

constexpr size_t kScratchBytes = size_t(8) << 20;   // KVQ_SCRATCH_BYTES
static_assert(kScratchBytes == KVQ_SCRATCH_BYTES, "header and library agree on the scratch size");
constexpr int kMaxDevices = 64;

// One copy per GPU the library runs on, held until the process ends.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this GPU's `scratch` (the host-side name of the
// array is not a device address), looked up once per device with that
// device current.
kvq_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return KVQ_ELAUNCH;
  if (dev >= kMaxDevices) return KVQ_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return KVQ_ELAUNCH;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KVQ_OK;
}

}  // namespace

extern "C" {

kvq_status kvq_decode_attn_noalloc(const kvq_decode_args* args, void* stream) {
  Plan pl;
  const kvq_status st = make_plan(args, &pl);
  if (st != KVQ_OK) return st;
  if (pl.ws_bytes > kScratchBytes) return KVQ_ESCRATCH;
  if (pl.ws_bytes > 0) {
    void* ws = nullptr;
    const kvq_status sa = scratch_address(&ws);
    if (sa != KVQ_OK) return sa;
    pl.p.ws = static_cast<float*>(ws);
  }
  return from_hip(kvq::launch_decode(pl.p, pl.GQ, static_cast<hipStream_t>(stream)));
}

kvq_status kvq_page_layout(int32_t n_kv_heads, int32_t d_h, int32_t group, int32_t bits,
                           int32_t page_tokens, int64_t out[5]) {
  if (!out) return KVQ_EINVAL;
  PageLayout L;
  const kvq_status st = page_layout(n_kv_heads, d_h, group, bits, page_tokens, &L);
  if (st != KVQ_OK) return st;
  out[0] = L.head_bytes;
  out[1] = L.kmeta_off;
  out[2] = L.vcodes_off;
  out[3] = L.vmeta_off;
  out[4] = L.page_bytes;
  return KVQ_OK;
}

kvq_status kvq_decode_attn_paged_workspace(const kvq_paged_args* args, size_t* bytes) {
  if (!bytes) return KVQ_EINVAL;
  Plan pl;
  const kvq_status st = make_paged_plan(args, &pl);
  if (st != KVQ_OK) return st;
  *bytes = pl.ws_bytes;
  return KVQ_OK;
}

kvq_status kvq_decode_attn_paged(const kvq_paged_args* args, void* stream) {
  Plan pl;
  const kvq_status st = make_paged_plan(args, &pl);
  if (st != KVQ_OK) return st;
  if (pl.ws_bytes > 0 && (!args->workspace || args->workspace_bytes < pl.ws_bytes))
    return KVQ_EWORKSPACE;
  return from_hip(kvq::launch_decode_paged(pl.p, pl.GQ, static_cast<hipStream_t>(stream)));
}

kvq_status kvq_pq_search(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t d_h, int32_t m,
                         int32_t bits, int32_t n_tok, int32_t top_k, const void* q, const void* centroids,
                         const void* codes, int64_t codes_stride, float* scores, int32_t* top_idx,
                         void* stream) {
  if (batch < 1 || n_kv_heads < 1 || n_q_heads < 1 || n_q_heads % n_kv_heads != 0) return KVQ_EINVAL;
  const int gq = n_q_heads / n_kv_heads;
  if (int64_t(batch) * n_kv_heads > 65535 || int64_t(batch) * n_q_heads > (int64_t(1) << 31))
    return KVQ_EUNSUPPORTED;
  if (!valid_d(d_h)) return KVQ_EUNSUPPORTED;
  if (m < 1 || d_h % m != 0 || (d_h / m) % 8 != 0 || 16 % m != 0) return KVQ_EUNSUPPORTED;
  if (bits < 1 || bits > 8) return KVQ_EINVAL;
  if (n_tok < 1 || n_tok > (1 << 24) || top_k < 1 || top_k > n_tok) return KVQ_EINVAL;
  if (!q || !centroids || !codes || !scores || !top_idx) return KVQ_EINVAL;
  if (codes_stride < int64_t(n_tok) * m) return KVQ_EINVAL;
  if (codes_stride & 15) return KVQ_EALIGN;
  for (const void* ptr : {q, centroids, codes, static_cast<const void*>(scores)})
    if (!aligned16(ptr)) return KVQ_EALIGN;
  if (reinterpret_cast<uintptr_t>(top_idx) & 3) return KVQ_EALIGN;
  const int GQ = kvq::head_block(gq);     // the scores kernel's head block (grid z)
  // one kernel when a head's scores fit in the 160 KB of LDS a gfx950
  // workgroup can hold (up to about 38K tokens), else scores then Top-k
  // through memory
  const bool fused = kvq::pq_fused_lds_bytes(n_tok, d_h, m, bits) <= 160 * 1024;
  if (!fused && kvq::pq_scores_lds_bytes(GQ, d_h, m, bits) > 64 * 1024) return KVQ_EUNSUPPORTED;
  kvq::PqParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.centroids = static_cast<const uint16_t*>(centroids);
  p.codes = static_cast<const uint8_t*>(codes);
  p.scores = scores;
  p.top_idx = top_idx;
  p.codes_stride = codes_stride;
  p.B = batch;
  p.Hq = n_q_heads;
  p.Hkv = n_kv_heads;
  p.gq = gq;
  p.D = d_h;
  p.m = m;
  p.bits = bits;
  p.n_tok = n_tok;
  p.top_k = top_k;
  p.chunk_tokens = 4096;
  return from_hip(kvq::launch_pq_search(p, GQ, fused, static_cast<hipStream_t>(stream)));
}

// Decode attention over a vector-quantized (codebook) cache: the token
// chunks and the workspace of a call.
static kvq_status vq_plan(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t d_h, int32_t rounds,
                          int32_t n_tok, kvq::VqParams* p, size_t* ws_bytes) {
  if (batch < 1 || n_kv_heads < 1 || n_q_heads < 1 || n_q_heads % n_kv_heads != 0) return KVQ_EINVAL;
  if (int64_t(batch) * n_kv_heads > 65535 || int64_t(batch) * n_q_heads > (int64_t(1) << 31))
    return KVQ_EUNSUPPORTED;
  if (!valid_d(d_h) || (rounds != 1 && rounds != 2)) return KVQ_EUNSUPPORTED;
  if (n_tok < 1 || n_tok > (1 << 24)) return KVQ_EINVAL;
  // chunks of at most kVqMaxChunk tokens; more (down to 256 tokens) when the
  // streams alone give fewer than 512 workgroups (two per CU)
  const int64_t streams = int64_t(batch) * n_kv_heads;
  int64_t nc = (int64_t(n_tok) + kvq::kVqMaxChunk - 1) / kvq::kVqMaxChunk;
  const int64_t want = std::min<int64_t>((512 + streams - 1) / streams, (int64_t(n_tok) + 255) / 256);
  nc = std::max(nc, want);
  int64_t chunk = (int64_t(n_tok) + nc - 1) / nc;
  chunk = std::min<int64_t>(kvq::kVqMaxChunk, (chunk + 63) / 64 * 64);
  nc = (int64_t(n_tok) + chunk - 1) / chunk;
  if (nc > kvq::kVqMaxChunks) return KVQ_EUNSUPPORTED;
  if (kvq::vq_lds_bytes(d_h, int(chunk)) + 4096 > 160 * 1024) return KVQ_EUNSUPPORTED;
  std::memset(p, 0, sizeof(*p));
  p->B = batch;
  p->Hq = n_q_heads;
  p->Hkv = n_kv_heads;
  p->gq = n_q_heads / n_kv_heads;
  p->D = d_h;
  p->R = rounds;
  p->n_tok = n_tok;
  p->chunk_tokens = int32_t(chunk);
  p->n_chunks = int32_t(nc);
  *ws_bytes = nc == 1 ? 0 : size_t(streams) * size_t(nc) * size_t(p->gq) * size_t(d_h + 2) * sizeof(float);
  return KVQ_OK;
}

kvq_status kvq_vq_decode_attn_workspace(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t d_h,
                                        int32_t rounds, int32_t n_tok, size_t* bytes) {
  if (!bytes) return KVQ_EINVAL;
  kvq::VqParams p;
  return vq_plan(batch, n_q_heads, n_kv_heads, d_h, rounds, n_tok, &p, bytes);
}

kvq_status kvq_vq_decode_attn(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t d_h, int32_t rounds,
                              int32_t n_tok, float sm_scale, const void* q, const void* k_codes,
                              const void* v_codes, int64_t codes_stride, const void* k_books,
                              const void* v_books, float* out, void* workspace, size_t workspace_bytes,
                              void* stream) {
  kvq::VqParams p;
  size_t need = 0;
  const kvq_status st = vq_plan(batch, n_q_heads, n_kv_heads, d_h, rounds, n_tok, &p, &need);
  if (st != KVQ_OK) return st;
  if (!std::isfinite(sm_scale)) return KVQ_EINVAL;
  if (!q || !k_codes || !v_codes || !k_books || !v_books || !out) return KVQ_EINVAL;
  if (codes_stride < int64_t(n_tok) * rounds * (d_h / 4)) return KVQ_EINVAL;
  if (codes_stride & 15) return KVQ_EALIGN;
  for (const void* ptr : {q, k_codes, v_codes, k_books, v_books})
    if (!aligned16(ptr)) return KVQ_EALIGN;
  if (reinterpret_cast<uintptr_t>(out) & 3) return KVQ_EALIGN;
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return KVQ_EWORKSPACE;
    if (!aligned16(workspace)) return KVQ_EALIGN;
  }
  p.q = static_cast<const uint16_t*>(q);
  p.k_codes = static_cast<const uint8_t*>(k_codes);
  p.v_codes = static_cast<const uint8_t*>(v_codes);
  p.k_books = static_cast<const uint16_t*>(k_books);
  p.v_books = static_cast<const uint16_t*>(v_books);
  p.out = out;
  p.ws = static_cast<float*>(workspace);
  p.codes_stride = codes_stride;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  return from_hip(kvq::launch_vq_decode(p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// One KIVI decode step (append, flushes, attention) from the cache state.
namespace {

struct KiviStep {
  kvq_kivi_cache next;       // the state after the step
  bool compact;              // move the window to row 0 first
  int32_t v_row, v_quant_row, v_dst_tok, k_row;
  bool flush_keys;           // quantize the R residual keys after the append
  int32_t flush_dst_tok;
  kvq_segment kseg, vseg;
  kvq_decode_args args;      // attention over `next` (pointers to q/out filled by the caller)
};

kvq_status kivi_plan_step(const kvq_kivi_cache* c, int32_t batch, int32_t n_q_heads, float sm_scale,
                          KiviStep* st) {
  if (!c || !st) return KVQ_EINVAL;
  const int64_t R = c->residual, G = c->group;
  if (c->bits != 2 && c->bits != 4 && c->bits != 8) return KVQ_EINVAL;
  if (G != 32 && G != 64 && G != 128) return KVQ_EINVAL;
  if (c->d_h != 64 && c->d_h != 128) return KVQ_EUNSUPPORTED;
  if (G > c->d_h || R < G || R % G != 0) return KVQ_EINVAL;
  if (c->n_streams < 1 || batch < 1 || c->n_streams % batch != 0) return KVQ_EINVAL;
  const int32_t hkv = c->n_streams / batch;
  if (n_q_heads < hkv || n_q_heads % hkv != 0) return KVQ_EINVAL;
  if (c->win_rows < 2 * R + 2 || c->reserved != 0) return KVQ_EINVAL;
  if (c->n_kq < 0 || c->r_k < 0 || c->r_k >= R || c->n_kq % G != 0) return KVQ_EINVAL;
  if (c->n_vq < 0 || c->r_v < 0 || c->r_v > R || c->v_start < 0 ||
      int64_t(c->v_start) + c->r_v > c->win_rows)
    return KVQ_EINVAL;
  if (int64_t(c->n_kq) + c->r_k != int64_t(c->n_vq) + c->r_v) return KVQ_EINVAL;
  if (int64_t(c->n_kq) + c->r_k + 1 > c->capacity) return KVQ_EINVAL;

  KiviStep& s = *st;
  s.next = *c;
  kvq_kivi_cache& n = s.next;
  // 1. window ring: with win_rows >= 2R + 2 the moved rows never overlap their source
  s.compact = int64_t(n.v_start) + n.r_v + 1 > n.win_rows;
  if (s.compact) n.v_start = 0;
  // 2. append, and the value-window overflow
  s.k_row = n.r_k;
  s.v_row = n.v_start + n.r_v;
  const bool quant = n.r_v + 1 > R;
  s.v_quant_row = quant ? n.v_start : -1;
  s.v_dst_tok = n.n_vq;
  n.r_k += 1;
  n.r_v += 1;
  if (quant) {
    n.n_vq += 1;
    n.v_start += 1;
    n.r_v -= 1;
  }
  // 3. key flush
  s.flush_keys = n.r_k == R;
  s.flush_dst_tok = n.n_kq;
  if (s.flush_keys) {
    n.n_kq += int32_t(R);
    n.r_k = 0;
  }
  // 4. attention over the new state
  s.kseg = kvq_segment{c->bits, 0, n.n_kq, 0, 0, 0};
  s.vseg = kvq_segment{c->bits, 0, n.n_vq, 0, 0, 0};
  kvq_decode_args& a = s.args;
  std::memset(&a, 0, sizeof(a));
  a.batch = batch;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = hkv;
  a.d_h = c->d_h;
  a.group = c->group;
  a.sm_scale = sm_scale;
  a.k_segs = &s.kseg;
  a.n_k_segs = n.n_kq > 0 ? 1 : 0;
  a.v_segs = &s.vseg;
  a.n_v_segs = n.n_vq > 0 ? 1 : 0;
  a.k_codes = c->k_codes; a.k_codes_stride = c->k_codes_stride;
  a.k_meta = c->k_meta;   a.k_meta_stride = c->k_meta_stride;
  a.v_codes = c->v_codes; a.v_codes_stride = c->v_codes_stride;
  a.v_meta = c->v_meta;   a.v_meta_stride = c->v_meta_stride;
  a.k_res = c->k_res; a.n_k_res = n.r_k; a.k_res_stride = c->k_res_stride;
  a.v_res = static_cast<const uint16_t*>(c->v_res) + int64_t(n.v_start) * c->d_h;
  a.n_v_res = n.r_v;
  a.v_res_stride = c->v_res_stride;
  return KVQ_OK;
}

}  // namespace

extern "C" {

kvq_status kvq_kivi_step_workspace(const kvq_kivi_cache* cache, int32_t batch, int32_t n_q_heads,
                                   size_t* bytes) {
  if (!bytes) return KVQ_EINVAL;
  KiviStep st;
  kvq_status r = kivi_plan_step(cache, batch, n_q_heads, 1.f, &st);
  if (r != KVQ_OK) return r;
  // the plan does not depend on q/out, but make_plan checks their alignment
  st.args.q = cache->k_res;
  st.args.out = static_cast<float*>(cache->v_res);
  return kvq_decode_attn_workspace(&st.args, bytes);
}

kvq_status kvq_kivi_step(kvq_kivi_cache* cache, int32_t batch, int32_t n_q_heads, float sm_scale,
                         const void* k_new, int64_t k_new_stride, const void* v_new,
                         int64_t v_new_stride, const void* q, float* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  KiviStep st;
  kvq_status r = kivi_plan_step(cache, batch, n_q_heads, sm_scale, &st);
  if (r != KVQ_OK) return r;
  const kvq_kivi_cache& c = *cache;
  const kvq_kivi_cache& n = st.next;
  if (!k_new || !v_new || !q || !out) return KVQ_EINVAL;
  st.args.q = q;
  st.args.out = out;
  st.args.workspace = workspace;
  st.args.workspace_bytes = workspace_bytes;
  // every check before the first launch
  Plan pl;
  r = make_plan(&st.args, &pl);
  if (r != KVQ_OK) return r;
  if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes)) return KVQ_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(k_new) & 15) || (reinterpret_cast<uintptr_t>(v_new) & 15) ||
      (k_new_stride & 7) || (v_new_stride & 7))
    return KVQ_EALIGN;
  if (k_new_stride < c.d_h || v_new_stride < c.d_h) return KVQ_EINVAL;

  // fused append + attention in one launch when the last wave of each
  // stream's single workgroup holds every token the append writes
  // (tokens the append writes: the new token N-1, key and value, and the
  // quantized value token with its pair partner).  With several head blocks
  // (grid z) every block's last wave performs the same append: the same bytes
  // from the same inputs, so each block reads what it wrote itself whatever
  // the order of the other blocks' identical stores.
  int32_t first_written = n.n_kq + st.k_row;
  if (st.v_quant_row >= 0) first_written = std::min(first_written, st.v_dst_tok & ~1);
  const bool fused = !st.compact && !st.flush_keys && pl.p.wg_per_stream == 1 && pl.p.n_bounds > 0 &&
                     pl.p.bounds[pl.p.waves_per_stream - 1] <= first_written;
  if (fused) {
    kvq::AppendParams& ap = pl.p.app;
    ap.k_new = static_cast<const uint16_t*>(k_new);
    ap.v_new = static_cast<const uint16_t*>(v_new);
    ap.k_res = static_cast<uint16_t*>(c.k_res);
    ap.v_res = static_cast<uint16_t*>(c.v_res);
    ap.v_codes = static_cast<uint8_t*>(c.v_codes);
    ap.v_meta = static_cast<uint8_t*>(c.v_meta);
    ap.k_new_stride = k_new_stride;
    ap.v_new_stride = v_new_stride;
    ap.k_res_stride = c.k_res_stride;
    ap.v_res_stride = c.v_res_stride;
    ap.v_codes_stride = c.v_codes_stride;
    ap.v_meta_stride = c.v_meta_stride;
    ap.bits = c.bits;
    ap.G = c.group;
    ap.D = c.d_h;
    ap.n_streams = c.n_streams;
    ap.k_row = st.k_row;
    ap.v_row = st.v_row;
    ap.v_quant_row = st.v_quant_row;
    ap.v_dst_tok = st.v_dst_tok;
    pl.p.fused_append = 1;
    r = from_hip(kvq::launch_decode(pl.p, pl.GQ, static_cast<hipStream_t>(stream)));
    if (r != KVQ_OK) return r;
    cache->last_launches = 1;
  } else {
  int32_t launches = 0;
  if (st.compact) {
    ++launches;
    r = kvq_residual_append(c.n_streams, c.d_h, c.r_v,
                            static_cast<const uint16_t*>(c.v_res) + int64_t(c.v_start) * c.d_h,
                            c.v_res_stride, c.d_h, c.v_res, c.v_res_stride, 0, stream);
    if (r != KVQ_OK) return r;
  }
  ++launches;
  r = kvq_decode_append(c.bits, c.group, c.n_streams, c.d_h, k_new, k_new_stride, v_new, v_new_stride,
                        c.k_res, c.k_res_stride, st.k_row, c.v_res, c.v_res_stride, st.v_row,
                        st.v_quant_row, c.v_codes, c.v_codes_stride, c.v_meta, c.v_meta_stride,
                        st.v_dst_tok, stream);
  if (r != KVQ_OK) return r;
  if (st.flush_keys) {
    ++launches;
    r = kvq_quantize_append(KVQ_KEYS, c.bits, c.group, c.n_streams, c.d_h, c.residual, c.k_res,
                            c.k_res_stride, c.d_h, nullptr, c.k_codes, c.k_codes_stride, c.k_meta,
                            c.k_meta_stride, st.flush_dst_tok, stream);
    if (r != KVQ_OK) return r;
  }
  r = from_hip(kvq::launch_decode(pl.p, pl.GQ, static_cast<hipStream_t>(stream)));
  if (r != KVQ_OK) return r;
  cache->last_launches = launches + (pl.p.wg_per_stream > 1 ? 2 : 1);
  }
  cache->n_kq = n.n_kq;
  cache->r_k = n.r_k;
  cache->n_vq = n.n_vq;
  cache->r_v = n.r_v;
  cache->v_start = n.v_start;
  return KVQ_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// WindowQuant window-level search.
namespace {

kvq_status search_shape(int32_t batch, int32_t n_text, int32_t n_visual, int32_t dim,
                        int32_t window_tokens, int64_t* n_windows, int64_t* n_chunks) {
  if (batch < 1 || n_text < 1 || window_tokens < 1 || n_visual < window_tokens) return KVQ_EINVAL;
  if (dim < 8 || dim % 8 != 0) return KVQ_EINVAL;
  if (dim > 4096 || batch > 65535) return KVQ_EUNSUPPORTED;
  *n_windows = n_visual / window_tokens;
  *n_chunks = kvq::search_chunks(n_text, int32_t(*n_windows), window_tokens);
  if (*n_chunks > (int64_t(1) << 30)) return KVQ_EUNSUPPORTED;
  return KVQ_OK;
}

}  // namespace

extern "C" {

kvq_status kvq_window_thresholds(float layer_similarity, float alpha, float* t_low, float* t_high) {
  if (!t_low || !t_high || !std::isfinite(layer_similarity) || !std::isfinite(alpha) || alpha == 0.f)
    return KVQ_EINVAL;
  const double s = layer_similarity, a = alpha;
  *t_low = float(std::expm1(a * s) / std::expm1(a));
  *t_high = float(std::expm1(-a * s) / std::expm1(-a));
  return KVQ_OK;
}

kvq_status kvq_window_search_workspace(int32_t batch, int32_t n_text, int32_t n_visual, int32_t dim,
                                       int32_t window_tokens, size_t* bytes) {
  if (!bytes) return KVQ_EINVAL;
  int64_t w, c;
  const kvq_status st = search_shape(batch, n_text, n_visual, dim, window_tokens, &w, &c);
  if (st != KVQ_OK) return st;
  *bytes = size_t(batch) * size_t(c) * size_t(dim) * sizeof(float);
  return KVQ_OK;
}

kvq_status kvq_window_search(int32_t batch, int32_t n_text, int32_t n_visual, int32_t dim,
                             const void* text, int64_t text_batch_stride, int64_t text_row_stride,
                             const void* visual, int64_t visual_batch_stride, int64_t visual_row_stride,
                             int32_t window_tokens, float t_low, float t_high, int32_t first_window_fp16,
                             float* scores, uint8_t* win_bits, void* workspace, size_t workspace_bytes,
                             void* stream) {
  int64_t n_windows, n_chunks;
  kvq_status st = search_shape(batch, n_text, n_visual, dim, window_tokens, &n_windows, &n_chunks);
  if (st != KVQ_OK) return st;
  if (!text || !visual || !win_bits || !std::isfinite(t_low) || !std::isfinite(t_high)) return KVQ_EINVAL;
  if (text_row_stride < dim || visual_row_stride < dim || text_batch_stride < 0 || visual_batch_stride < 0)
    return KVQ_EINVAL;
  if ((reinterpret_cast<uintptr_t>(text) & 15) || (reinterpret_cast<uintptr_t>(visual) & 15) ||
      (reinterpret_cast<uintptr_t>(scores) & 3) || (reinterpret_cast<uintptr_t>(workspace) & 15) ||
      (text_row_stride & 7) || (visual_row_stride & 7) || (text_batch_stride & 7) ||
      (visual_batch_stride & 7))
    return KVQ_EALIGN;
  const size_t need = size_t(batch) * size_t(n_chunks) * size_t(dim) * sizeof(float);
  if (!workspace || workspace_bytes < need) return KVQ_EWORKSPACE;
  kvq::SearchParams p{};
  p.text = static_cast<const uint16_t*>(text);
  p.visual = static_cast<const uint16_t*>(visual);
  p.text_batch_stride = text_batch_stride;
  p.text_row_stride = text_row_stride;
  p.visual_batch_stride = visual_batch_stride;
  p.visual_row_stride = visual_row_stride;
  p.ws = static_cast<float*>(workspace);
  p.scores = scores;
  p.win_bits = win_bits;
  p.B = batch;
  p.N = n_text;
  p.D = dim;
  p.S = window_tokens;
  p.n_windows = int32_t(n_windows);
  p.chunks_per_window = kvq::search_chunks_per_window(window_tokens);
  p.n_chunks = int32_t(n_chunks);
  p.first_window_fp16 = first_window_fp16 ? 1 : 0;
  p.t_low = t_low;
  p.t_high = t_high;
  return from_hip(kvq::launch_search(p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
