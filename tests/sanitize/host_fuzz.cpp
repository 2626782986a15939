// Host-side fuzzing of the library's planning and argument checks, built
// with AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_host_sanitize.py).
//
// Every call here stays on the host: the workspace queries only plan, and
// the launching entry points are only called with arguments that fail a
// check made before anything is enqueued (a workspace one byte too small,
// a null required pointer, an out-of-range field).  Device pointers are fake
// aligned addresses that the host code never dereferences.  Exit status 0
// means every call returned a defined status and the sanitizers found
// nothing (they abort the process otherwise).
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "kvq.h"

namespace {

std::mt19937_64 rng(20261202);
int64_t uni(int64_t lo, int64_t hi) { return std::uniform_int_distribution<int64_t>(lo, hi)(rng); }
template <class T> T pick(std::initializer_list<T> v) { return *(v.begin() + uni(0, int64_t(v.size()) - 1)); }
void* fake(int64_t align = 256) { return reinterpret_cast<void*>(uintptr_t(uni(1, 1 << 20)) * uintptr_t(align)); }

int64_t n_calls = 0, n_ok = 0;
void count(kvq_status s) {
  ++n_calls;
  if (s == KVQ_OK) ++n_ok;
  if (int(s) < 0 || int(s) > 6 || !kvq_strerror(int32_t(s))) {
    std::fprintf(stderr, "undefined status %d\n", int(s));
    std::exit(2);
  }
}

// runs of `total` tokens: mostly well formed, sometimes with a wrong field
std::vector<kvq_segment> runs(int total, int G, bool keys) {
  std::vector<kvq_segment> v;
  int t = 0;
  const int n = int(uni(0, 9));
  for (int i = 0; i < n && t < total; ++i) {
    kvq_segment s{};
    s.bits = pick({2, 4, 8, 16, 16, 2, 3});
    int len = int(uni(1, total - t));
    if (keys && s.bits != 16 && uni(0, 3)) len = std::max(G, len / G * G);
    if (!keys && s.bits != 16 && uni(0, 3)) len = std::max(2, len & ~1);
    if (t + len > total) len = total - t;
    s.tok_begin = uni(0, 20) ? t : t + int(uni(-3, 3));
    s.n_tok = len;
    s.reserved = uni(0, 30) ? 0 : 1;
    s.code_off = uni(0, 1 << 20) * (uni(0, 20) ? 16 : 1);
    s.meta_off = uni(0, 1 << 20) * (uni(0, 20) ? 16 : 1);
    v.push_back(s);
    t += len;
  }
  return v;
}

void fuzz_decode() {
  kvq_decode_args a{};
  a.batch = int32_t(pick<int64_t>({1, 2, 4, 16, 64, 0, -1, 70000}));
  a.n_kv_heads = int32_t(pick<int64_t>({1, 2, 4, 8, 32, 0}));
  a.n_q_heads = a.n_kv_heads * int32_t(pick<int64_t>({1, 2, 3, 4, 7, 8, 16, 32, 71})) + (uni(0, 15) ? 0 : 1);
  a.d_h = int32_t(pick<int64_t>({64, 128, 128, 96, 0}));
  a.group = int32_t(pick<int64_t>({32, 64, 128, 16}));
  a.sm_scale = pick<float>({0.088f, 1.0f, 0.0f, NAN, INFINITY});
  const int n_k_q = int(uni(0, 40000)), n_k_res = int(uni(0, 300));
  const int total = n_k_q + n_k_res;
  std::vector<kvq_segment> ks = runs(n_k_q, std::max<int32_t>(a.group, 1), true);
  int covered = 0;
  for (auto& s : ks) covered = std::max(covered, s.tok_begin + s.n_tok);
  a.n_k_res = uni(0, 10) ? total - covered : int32_t(uni(-2, 400));
  const int n_v_res = int(uni(0, 400));
  std::vector<kvq_segment> vs = runs(std::max(0, total - n_v_res), std::max<int32_t>(a.group, 1), false);
  int vcov = 0;
  for (auto& s : vs) vcov = std::max(vcov, s.tok_begin + s.n_tok);
  a.n_v_res = uni(0, 10) ? total - vcov : int32_t(uni(-2, 400));
  a.k_segs = ks.empty() ? nullptr : ks.data();
  a.n_k_segs = uni(0, 20) ? int32_t(ks.size()) : int32_t(uni(-1, 12));
  a.v_segs = vs.empty() ? nullptr : vs.data();
  a.n_v_segs = uni(0, 20) ? int32_t(vs.size()) : int32_t(uni(-1, 12));
  if (a.n_k_segs > int32_t(ks.size()) && !ks.empty()) a.n_k_segs = int32_t(ks.size());
  if (a.n_v_segs > int32_t(vs.size()) && !vs.empty()) a.n_v_segs = int32_t(vs.size());
  a.q = uni(0, 30) ? fake(uni(0, 10) ? 256 : 2) : nullptr;
  a.k_codes = fake(); a.k_meta = fake(); a.v_codes = fake(); a.v_meta = fake();
  a.k_codes_stride = uni(0, 1 << 22) * 16; a.k_meta_stride = uni(0, 1 << 22) * 16;
  a.v_codes_stride = uni(0, 1 << 22) * 16; a.v_meta_stride = uni(0, 1 << 22) * 16;
  a.k_res = fake(); a.v_res = fake();
  a.k_res_stride = uni(0, 1 << 16) * (uni(0, 10) ? 8 : 3);
  a.v_res_stride = uni(0, 1 << 16) * (uni(0, 10) ? 8 : 3);
  a.out = static_cast<float*>(fake());
  a.split_tokens = int32_t(pick<int64_t>({0, 0, 64, 256, 1000, 1 << 20, -5}));
  size_t need = 0;
  const kvq_status s = kvq_decode_attn_workspace(&a, &need);
  count(s);
  if (s == KVQ_OK && need > 0) {
    // checks pass, the workspace is one byte short: refused before a launch
    a.workspace = fake();
    a.workspace_bytes = need - 1;
    const kvq_status r = kvq_decode_attn(&a, nullptr);
    count(r);
    if (r != KVQ_EWORKSPACE) { std::fprintf(stderr, "short workspace not refused: %d\n", int(r)); std::exit(3); }
    a.workspace = nullptr;
    a.workspace_bytes = need;
    count(kvq_decode_attn(&a, nullptr));
    if (need > KVQ_SCRATCH_BYTES) {
      const kvq_status n = kvq_decode_attn_noalloc(&a, nullptr);
      count(n);
      if (n != KVQ_ESCRATCH) { std::fprintf(stderr, "oversized no-alloc call not refused: %d\n", int(n)); std::exit(4); }
    }
  }
}

void fuzz_paged() {
  kvq_paged_args a{};
  a.batch = int32_t(pick<int64_t>({1, 3, 32, 256, 300, 0}));
  a.n_kv_heads = int32_t(pick<int64_t>({1, 2, 8, 32}));
  a.n_q_heads = a.n_kv_heads * int32_t(pick<int64_t>({1, 2, 4, 7, 8, 16})) + (uni(0, 15) ? 0 : 1);
  a.d_h = int32_t(pick<int64_t>({64, 128, 80}));
  a.group = int32_t(pick<int64_t>({32, 64, 128}));
  a.bits = int32_t(pick<int64_t>({2, 4, 8, 5}));
  a.sm_scale = 0.088f;
  a.page_tokens = int32_t(pick<int64_t>({64, 128, 256, 1024, 100, 0}));
  a.q = fake(); a.pages = fake(); a.block_table = static_cast<const int32_t*>(fake());
  a.page_bytes = uni(1, 1 << 22) * 16;
  a.max_pages = int32_t(uni(0, 200));
  std::vector<int32_t> len(size_t(std::max(a.batch, 0)) * 4);
  for (int b = 0; b < a.batch; ++b) {
    const int PT = std::max<int32_t>(a.page_tokens, 1);
    int n_kq = int(uni(0, std::min<int64_t>(int64_t(a.max_pages) * PT, 1 << 16)));
    if (uni(0, 5)) n_kq = n_kq / std::max<int32_t>(a.group, 1) * std::max<int32_t>(a.group, 1);
    int n_vq = int(uni(0, n_kq));
    const int n_kres = int(uni(0, 200));
    len[4 * b] = n_kq; len[4 * b + 1] = n_vq; len[4 * b + 2] = n_kres;
    len[4 * b + 3] = uni(0, 20) ? n_kq + n_kres - n_vq : int32_t(uni(-5, 500));
  }
  a.lengths = len.empty() ? nullptr : len.data();
  a.lengths_dev = static_cast<const int32_t*>(fake());
  a.k_res = fake(); a.v_res = fake();
  a.k_res_stride = uni(0, 1 << 16) * 8; a.v_res_stride = uni(0, 1 << 16) * 8;
  a.out = static_cast<float*>(fake());
  size_t need = 0;
  const kvq_status s = kvq_decode_attn_paged_workspace(&a, &need);
  count(s);
  if (s == KVQ_OK && need > 0) {
    a.workspace = fake();
    a.workspace_bytes = need - 1;
    const kvq_status r = kvq_decode_attn_paged(&a, nullptr);
    count(r);
    if (r != KVQ_EWORKSPACE) { std::fprintf(stderr, "paged short workspace not refused: %d\n", int(r)); std::exit(5); }
  }
  int64_t out[5];
  count(kvq_page_layout(a.n_kv_heads, a.d_h, a.group, a.bits, a.page_tokens, uni(0, 20) ? out : nullptr));
}

void fuzz_kivi() {
  kvq_kivi_cache c{};
  c.bits = int32_t(pick<int64_t>({2, 4, 8, 3}));
  c.group = int32_t(pick<int64_t>({32, 64, 128}));
  c.residual = c.group * int32_t(uni(0, 8));
  c.n_streams = int32_t(pick<int64_t>({1, 4, 64, 512, 0}));
  c.d_h = int32_t(pick<int64_t>({64, 128}));
  c.capacity = int32_t(uni(0, 70000));
  c.win_rows = 2 * c.residual + int32_t(uni(-2, 10));
  c.reserved = uni(0, 30) ? 0 : 7;
  c.k_codes = fake(); c.k_meta = fake(); c.v_codes = fake(); c.v_meta = fake(); c.k_res = fake(); c.v_res = fake();
  c.k_codes_stride = uni(0, 1 << 22) * 16; c.k_meta_stride = uni(0, 1 << 22) * 16;
  c.v_codes_stride = uni(0, 1 << 22) * 16; c.v_meta_stride = uni(0, 1 << 22) * 16;
  c.k_res_stride = uni(0, 1 << 16) * 8; c.v_res_stride = uni(0, 1 << 16) * 8;
  c.n_kq = int32_t(uni(0, c.capacity + 10)) / std::max<int32_t>(c.group, 1) * std::max<int32_t>(c.group, 1);
  c.r_k = int32_t(uni(0, c.residual));
  c.n_vq = int32_t(uni(0, c.n_kq + c.r_k));
  c.r_v = uni(0, 10) ? c.n_kq + c.r_k - c.n_vq : int32_t(uni(-3, 300));
  c.v_start = int32_t(uni(0, std::max(c.win_rows, 1)));
  const int32_t hkv = int32_t(pick<int64_t>({1, 2, 4}));
  const int32_t batch = c.n_streams / hkv;
  const int32_t hq = hkv * int32_t(pick<int64_t>({1, 2, 4, 8, 9}));
  size_t need = 0;
  count(kvq_kivi_step_workspace(&c, batch, hq, &need));
  // a step with a null query is refused before anything is enqueued
  count(kvq_kivi_step(&c, batch, hq, 0.088f, fake(), c.d_h, fake(), c.d_h, nullptr,
                      static_cast<float*>(fake()), fake(), 1 << 30, nullptr));
}

void fuzz_misc() {
  float lo = 0, hi = 0;
  count(kvq_window_thresholds(pick<float>({0.5f, -2.f, 0.f, NAN, INFINITY}), pick<float>({1.f, 0.f, -3.f, NAN, 40.f}),
                              &lo, uni(0, 10) ? &hi : nullptr));
  size_t b = 0;
  count(kvq_window_search_workspace(int32_t(uni(-1, 70)), int32_t(uni(-1, 5000)), int32_t(uni(-1, 1 << 20)),
                                    int32_t(pick<int64_t>({64, 3584, 100, 0})), int32_t(pick<int64_t>({256, 64, 0, 7})), &b));
  count(kvq_vq_decode_attn_workspace(int32_t(uni(-1, 64)), int32_t(uni(-1, 64)), int32_t(uni(-1, 64)),
                                     int32_t(pick<int64_t>({64, 128, 96})), int32_t(uni(-1, 3)), int32_t(uni(-1, 1 << 20)), &b));
  // launching entry points with a required pointer missing
  count(kvq_quantize_append(int32_t(uni(-1, 2)), int32_t(pick<int64_t>({2, 4, 8, 16})), 32, int32_t(uni(1, 64)),
                            128, int32_t(uni(0, 4096)), nullptr, 1 << 20, 128, nullptr, fake(), 1 << 20, fake(),
                            1 << 20, int32_t(uni(0, 100)), nullptr));
  count(kvq_residual_append(int32_t(uni(1, 64)), 128, int32_t(uni(1, 64)), nullptr, 1 << 20, 128, fake(), 1 << 20,
                            int32_t(uni(0, 100)), nullptr));
  count(kvq_decode_append(2, 32, int32_t(uni(1, 64)), 128, nullptr, 128, fake(), 128, fake(), 1 << 14, 0, fake(),
                          1 << 14, 0, int32_t(uni(-1, 4)), fake(), 1 << 20, fake(), 1 << 20, int32_t(uni(0, 100)),
                          nullptr));
  std::vector<uint8_t> wb(size_t(uni(0, 300)));
  for (auto& x : wb) x = uint8_t(pick<int64_t>({2, 4, 8, 16, 5}));
  count(kvq_reorder_windows(wb.empty() ? nullptr : wb.data(), int32_t(wb.size()), int32_t(pick<int64_t>({256, 64, 0})),
                            32, 128, nullptr, static_cast<kvq_segment*>(fake()), static_cast<int32_t*>(fake()),
                            static_cast<int32_t*>(fake()), nullptr));
  for (int32_t st = -3; st < 10; ++st) count(kvq_strerror(st) ? KVQ_OK : KVQ_EINVAL);
}

}  // namespace

int main(int argc, char** argv) {
  const int64_t iters = argc > 1 ? std::atoll(argv[1]) : 4000;
  if (kvq_abi_version() != KVQ_ABI_VERSION) return 1;
  for (int64_t i = 0; i < iters; ++i) {
    fuzz_decode();
    fuzz_paged();
    fuzz_kivi();
    fuzz_misc();
  }
  std::printf("host fuzz: %lld calls, %lld accepted\n", (long long)n_calls, (long long)n_ok);
  return 0;
}
