/*
 * kvq.h -- C ABI of an MI355X (gfx950) library for decode-step attention over
 * a low-bit quantized KV cache.
 *
 * What is computed (the sources of the method):
 *   - KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache
 *     (papercache.org note on arXiv 2402.02750): asymmetric round-to-nearest
 *     Q(X) = round((X - z)/s), X' = Q*s + z; keys quantized per channel over
 *     groups of G tokens, values per token over groups of G channels; the most
 *     recent tokens stay in an fp16 residual; decode logits are the
 *     concatenation of the grouped part and the residual part under one
 *     softmax (sections "How it works", "Method details", Algorithm 1).
 *   - WindowQuant: Mixed-Precision KV Cache Quantization Based on Window-Level
 *     Similarity for VLMs Inference Optimization (ACM TACO): windows of S
 *     tokens get 8/4/2 bits (or stay fp16), windows of equal width are
 *     reordered to sit together, decode runs Q.K^T per width block, one
 *     softmax, per-block A.V summed (Sec. 3.1, 3.3.1, Eq. 12-16).
 *   - The split of the context across workgroups with a final merge of the
 *     partial softmax states follows the FlashDecoding dataflow that the
 *     VQ-LLM note (arXiv 2503.02236, reference [10]) describes.
 *
 * Conventions for every call:
 *   - All device pointers are plain HIP device addresses; the caller allocates
 *     and frees every buffer (cache arenas, residuals, query, output,
 *     workspace).  The library never allocates, frees or synchronizes.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on that stream and returns.
 *   - Arguments are checked on the host before anything is enqueued; on any
 *     error the call returns a status other than KVQ_OK and no device memory
 *     is touched.  Nothing aborts and nothing is thrown across the ABI.
 *   - No global mutable state: calls are re-entrant.  Calls that write the
 *     same buffers must be ordered by the caller (same stream or events).
 *   - A "stream" of the cache (not to be confused with a HIP stream) is one
 *     (batch b, kv head h) sequence; its index is b * n_kv_heads + h.
 *   - fp16 means IEEE binary16 stored as 16-bit words.
 *
 * Cache layout (not given by the pages; fixed here and part of the ABI).
 * The cache of each stream is a list of runs ("segments"), each holding
 * consecutive tokens at one bit width b, plus an fp16 residual.
 *   Code arena, keys, b in {2,4,8}: one row of RB = d_h*b/8 bytes per token,
 *     row t of the run at byte code_off + t*RB.  The code of channel c sits in
 *     byte floor(c*b/8) at bit (c*b) mod 8, low bits first.
 *   Code arena, values, b in {2,4,8}: tokens 2p and 2p+1 of the run share a
 *     block of 2*RB bytes at byte code_off + p*2*RB, made of RB/2
 *     little-endian 32-bit words; word w holds bytes 2w, 2w+1 of token 2p's
 *     row (the key row format) in its low 16 bits and the same two bytes of
 *     token 2p+1's row in its high 16 bits.
 *   Code arena, b = 16 (keys and values): rows of d_h fp16 values.
 *   Meta arena: (scale, zero) pairs of two fp16 values, 4 bytes per pair,
 *     starting at byte meta_off of the run.  Keys: the pair of group j
 *     (tokens jG..jG+G-1 of the run) and channel c has index j*d_h + c.
 *     Values: the pair of token t and channel group g (channels gG..gG+G-1)
 *     has index ((t/2)*(d_h/G) + g)*2 + (t mod 2).  b = 16 runs have no meta.
 *   Residual: fp16 rows of d_h values, row i of a stream at element
 *     stream*res_stride + i*d_h.
 *
 * Quantizer (bit-exact contract): for each group, in IEEE fp32 on the fp16
 * inputs, mn = min + 0, mx = max + 0 (zero extrema are +0), s32 = (mx - mn) /
 * (2^b - 1) (one correctly rounded division), s = fp16(s32) (round to
 * nearest even), z = fp16(mn) (exact); codes are 0 when s == 0, else
 * clamp(rint((x - z) / s), 0, 2^b - 1) with z, s widened from fp16, one fp32 subtraction and one correctly rounded
 * fp32 division, rint rounding half to even.  The stored (s, z) are the ones
 * used to encode, so X' = Q*s + z decodes what was encoded.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 1

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_EINVAL = 1,       /* argument out of range or inconsistent */
  KVQ_EALIGN = 2,       /* pointer, offset or stride not aligned as required */
  KVQ_EUNSUPPORTED = 3, /* well-formed, but not a shape this library runs */
  KVQ_EWORKSPACE = 4,   /* workspace missing or smaller than required */
  KVQ_ELAUNCH = 5,      /* the HIP runtime refused a kernel launch */
  KVQ_ESCRATCH = 6      /* kvq_decode_attn_noalloc: more than KVQ_SCRATCH_BYTES needed */
} kvq_status;

/* Which half of the cache a quantize call writes. */
enum { KVQ_KEYS = 0, KVQ_VALUES = 1 };

/* One run of consecutive cache tokens at one bit width.  The runs of a cache
 * are listed in token order: run i starts at the token where run i-1 ends. */
typedef struct kvq_segment {
  int32_t bits;      /* 16, 8, 4 or 2                                          */
  int32_t tok_begin; /* first token of the run, in attention (stored) order    */
  int32_t n_tok;     /* tokens in the run                                      */
  int32_t reserved;  /* must be 0                                              */
  int64_t code_off;  /* byte offset of the run in each stream's code arena     */
  int64_t meta_off;  /* byte offset of the run in each stream's meta arena     */
} kvq_segment;

/* ABI version of the loaded library (KVQ_ABI_VERSION at build time). */
int32_t kvq_abi_version(void);

/* Static, human-readable name of a status; never NULL. */
const char* kvq_strerror(int32_t status);

/*
 * kvq_quantize_append -- quantize n_tok fp16 rows of every stream, pack them
 * and append them to one run of the cache (KIVI GroupQuant / KeyQuant and the
 * decode-time flushes of Algorithm 1; WindowQuant per-window quantization of
 * reordered windows, Sec. 3.3.1 and Eq. 14-16).
 *
 *   which      KVQ_KEYS: per-channel groups of `group` consecutive tokens;
 *              requires n_tok % group == 0 and dst_tok % group == 0.
 *              KVQ_VALUES: per-token groups of `group` consecutive channels;
 *              any n_tok >= 1 and any dst_tok >= 0.
 *   bits       2, 4 or 8; or 16 = copy the rows unchanged (no meta written).
 *   group      G in {32, 64, 128}; values need G <= d_h.
 *   n_streams  B * Hkv (>= 1).     d_h  64 or 128.     n_tok >= 0 (0 = no-op).
 *   src        fp16 rows; row i of stream s at element
 *              s*src_stream_stride + r*src_row_stride, r = src_rows ? src_rows[i] : i.
 *              Both strides are multiples of 8 elements, src_row_stride >= d_h.
 *   src_rows   NULL, or device int32 [n_tok] of source row indices (gather, e.g.
 *              the row list of kvq_reorder_windows).  Indices are not checked
 *              on the device: each must address a row inside the caller's
 *              buffer.
 *   codes      device pointer to the run's first byte (arena + code_off) of
 *              stream 0; stream s at codes + s*codes_stream_stride bytes.
 *   meta       same for the (scale, zero) pairs (ignored for bits 16).
 *   dst_tok    tokens already in the run; new token i becomes run token
 *              dst_tok + i.  For values, a token sharing a pair block with an
 *              existing token only writes its own 16-bit halves; when the last
 *              appended token has an even index, the halves and (scale, zero)
 *              pair of the next (not yet written) token are set to zero, so a
 *              run of odd length never exposes uninitialized bytes to decode.
 * Alignment: src, codes, meta and the stream strides are multiples of 16 bytes.
 * Writes the bytes of the appended tokens and their meta pairs (and, as
 * above, zeroes the unwritten pair partner of a last even-index value token).
 */
kvq_status kvq_quantize_append(int32_t which, int32_t bits, int32_t group,
                               int32_t n_streams, int32_t d_h, int32_t n_tok,
                               const void* src, int64_t src_stream_stride,
                               int64_t src_row_stride, const int32_t* src_rows,
                               void* codes, int64_t codes_stream_stride,
                               void* meta, int64_t meta_stream_stride,
                               int32_t dst_tok, void* stream);

/*
 * kvq_residual_append -- copy n_rows fp16 rows of every stream into the fp16
 * residual at rows dst_row..dst_row+n_rows-1 (KIVI Algorithm 1, Decoding: the
 * new key and value rows are appended to the full-precision residuals).
 *   src: row r of stream s at element s*src_stream_stride + r*src_row_stride.
 *   dst: row i of stream s at element s*dst_stream_stride + i*d_h.
 * Strides are in fp16 elements, multiples of 8; pointers 16-byte aligned.
 */
kvq_status kvq_residual_append(int32_t n_streams, int32_t d_h, int32_t n_rows,
                               const void* src, int64_t src_stream_stride,
                               int64_t src_row_stride, void* dst,
                               int64_t dst_stream_stride, int32_t dst_row,
                               void* stream);

/*
 * kvq_decode_append -- one decode step's cache append in one launch (KIVI
 * Algorithm 1, Decoding): for every stream, the new key row goes to row
 * k_row of the key residual, the new value row to row v_row of the value
 * window, and, when v_quant_row >= 0, value-window row v_quant_row (the new
 * value row itself if v_quant_row == v_row) is quantized per token and
 * appended to the value run as token v_dst_tok -- the same bytes as
 * kvq_quantize_append(KVQ_VALUES, bits, group, ..., n_tok = 1, dst_tok =
 * v_dst_tok) of that row, including the zeroed pair partner at an even index.
 * Key-residual flushes (every R steps) stay kvq_quantize_append(KVQ_KEYS).
 *   bits 2, 4 or 8; group in {32, 64, 128}, group <= d_h; d_h 64 or 128.
 *   k_new, v_new   fp16 [n_streams] rows, stream s at element s*new_stride.
 *   k_res, v_res   fp16 residual / window; row i of stream s at element
 *                  s*res_stride + i*d_h.
 *   v_codes, v_meta   the value run's first byte (arena + offset) of stream 0;
 *                  stream s at + s*stride bytes (ignored if v_quant_row < 0).
 * Strides in fp16 elements are multiples of 8, byte strides and pointers
 * multiples of 16.  Rows and tokens are not range-checked on the device: they
 * must address rows inside the caller's buffers.
 */
kvq_status kvq_decode_append(int32_t bits, int32_t group, int32_t n_streams, int32_t d_h,
                             const void* k_new, int64_t k_new_stride,
                             const void* v_new, int64_t v_new_stride,
                             void* k_res, int64_t k_res_stride, int32_t k_row,
                             void* v_res, int64_t v_res_stride, int32_t v_row,
                             int32_t v_quant_row,
                             void* v_codes, int64_t v_codes_stride,
                             void* v_meta, int64_t v_meta_stride, int32_t v_dst_tok,
                             void* stream);

/*
 * kvq_reorder_windows -- WindowQuant window reorder (Sec. 3.3.1-3.3.2): a
 * stable sort of the windows by bit width, widest first (16, 8, 4, 2; equal
 * widths keep their original order), and the run table of the reordered cache.
 *
 *   win_bits       device uint8 [n_windows], each 16, 8, 4 or 2.
 *   n_windows      1..65536.   window_tokens  S, a multiple of `group`
 *                  (and even).   group, d_h   as for kvq_quantize_append.
 *   perm           device int32 [n_windows]: perm[new] = old window index.
 *   segs           device kvq_segment [4]: one run per width present, in the
 *                  order 16, 8, 4, 2; tok_begin = first reordered token of the
 *                  run; code_off / meta_off: runs are laid out one after the
 *                  other in each stream's arena, each starting at the previous
 *                  run's end rounded up to 256 bytes (codes and meta
 *                  separately).  Code bytes of a run: n_tok*d_h*b/8 (b < 16) or
 *                  n_tok*d_h*2 (b = 16); meta bytes: n_tok*(d_h/G)*4 (b < 16)
 *                  or 0.
 *   n_segs         device int32 [1]: number of runs, or -1 when a window
 *                  width is not one of 16/8/4/2 (then perm, segs and
 *                  row_gather hold no result).
 *   row_gather     NULL, or device int32 [n_windows*window_tokens]: the source
 *                  token of every reordered token, perm[w]*S + i at w*S + i.
 * The decode step applies no mask, so the reorder does not change its output
 * (Eq. 12-13); the prefill (masked) must run before it (Sec. 3.3.4).
 */
kvq_status kvq_reorder_windows(const uint8_t* win_bits, int32_t n_windows,
                               int32_t window_tokens, int32_t group, int32_t d_h,
                               int32_t* perm, kvq_segment* segs, int32_t* n_segs,
                               int32_t* row_gather, void* stream);

/*
 * Decode attention arguments.  For every batch row b and query head hq (kv
 * head h = hq / (n_q_heads / n_kv_heads), contiguous grouping), with the N
 * cache tokens of stream (b, h):
 *   logit_t = sm_scale * <q[b][hq], K'_t>,  p = softmax(logit) over all N,
 *   out[b][hq] = sum_t p_t V'_t,
 * where K'_t is the dequantized key of token t when t lies in a key run
 * (Q*s + z) or the fp16 residual key row t - n_Kq otherwise (n_Kq = tokens
 * in all key runs), and likewise V'_t with the value runs and residual.  This
 * is KIVI's A = Concat([A_g, A_r]) under one softmax, t_O = A_g Q(X_Vg) +
 * A_r X_Vr, with keys and values flushed at different token counts, and
 * WindowQuant's per-width block decode (Sec. 3.3.1).  No mask is applied.
 */
typedef struct kvq_decode_args {
  int32_t batch;          /* B >= 1                                              */
  int32_t n_q_heads;      /* Hq, a multiple of n_kv_heads (any ratio: MHA, GQA, MQA) */
  int32_t n_kv_heads;     /* Hkv >= 1                                            */
  int32_t d_h;            /* 64 or 128                                           */
  int32_t group;          /* G of the quantized runs (32, 64, 128; <= d_h)       */
  float sm_scale;         /* logit scale, e.g. 1/sqrt(d_h)                       */
  const void* q;          /* fp16 [B][Hq][d_h], contiguous                       */
  const kvq_segment* k_segs; /* HOST array of key runs, in token order          */
  int32_t n_k_segs;       /* 0..8                                                */
  const kvq_segment* v_segs; /* HOST array of value runs, in token order        */
  int32_t n_v_segs;       /* 0..8                                                */
  const void* k_codes;  int64_t k_codes_stride;  /* arena base, bytes/stream    */
  const void* k_meta;   int64_t k_meta_stride;
  const void* v_codes;  int64_t v_codes_stride;
  const void* v_meta;   int64_t v_meta_stride;
  const void* k_res;    int32_t n_k_res;  int64_t k_res_stride; /* fp16 elems  */
  const void* v_res;    int32_t n_v_res;  int64_t v_res_stride;
  float* out;             /* fp32 [B][Hq][d_h]                                   */
  void* workspace;        /* device scratch, see kvq_decode_attn_workspace       */
  size_t workspace_bytes;
  int32_t split_tokens;   /* tokens per workgroup; 0 = chosen by the library     */
} kvq_decode_args;

/*
 * Bytes of workspace kvq_decode_attn needs for these arguments (it depends
 * on the shapes, the runs and split_tokens, not on the pointers; 0 when each
 * stream fits one workgroup, and then workspace may be NULL).  The workspace
 * holds per-workgroup partial softmax states; it needs no initialization,
 * its contents are scratch after the call, and calls that share one must
 * not overlap.
 */
kvq_status kvq_decode_attn_workspace(const kvq_decode_args* args, size_t* bytes);

/*
 * kvq_decode_attn -- one decode step of attention for every (b, hq).
 * A value run of odd length must have the missing pair partner's (scale,
 * zero) finite (kvq_quantize_append leaves it zero).
 * Checks (all before any launch): shapes as documented above; runs in token
 * order with sum(k n_tok) + n_k_res == sum(v n_tok) + n_v_res = N >= 1;
 * key runs with b < 16 hold whole groups (n_tok % G == 0); code_off and
 * meta_off multiples of 16; pointers and byte strides multiples of 16;
 * residual strides multiples of 8 elements; workspace large enough.
 * Reads the cache, q and the residuals; writes out and the workspace only.
 */
kvq_status kvq_decode_attn(const kvq_decode_args* args, void* stream);

/*
 * kvq_decode_attn_noalloc -- kvq_decode_attn for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc): the same checks, kernels and result, but the
 * partial softmax states go to the library's own device array of
 * KVQ_SCRATCH_BYTES (one per GPU, held until the process ends) instead of
 * args->workspace, which is ignored (workspace_bytes too).  Returns
 * KVQ_ESCRATCH, touching nothing, when kvq_decode_attn_workspace would
 * report more than KVQ_SCRATCH_BYTES.  Calls no allocating routine; the
 * first call on a device looks up that device's array address (with the
 * device current) and keeps it.  Every call on one GPU shares that array:
 * calls that overlap on one GPU (other HIP streams, other threads) race and
 * must be ordered by the caller; the array needs no initialization (each
 * call writes every partial state it reads).
 */
#define KVQ_SCRATCH_BYTES (8u << 20)
kvq_status kvq_decode_attn_noalloc(const kvq_decode_args* args, void* stream);

/*
 * Paged, ragged cache (the serving layout).  The KIVI note's outlook pairs
 * the method with PagedAttention ("Conclusion and outlook"); the VQ-LLM note
 * measures paged FlashDecoding baselines.  Every sequence b has its own
 * lengths, and its quantized tokens live in fixed-size pages taken from one
 * pool in any order, listed by a block table.
 *
 * kvq_page_layout -- the byte layout of one page: page_tokens (PT) tokens of
 * one sequence for all n_kv_heads kv heads, keys and values at one bit width.
 * Kv head h's block starts at h*head_bytes; inside it:
 *   key codes   at 0:          PT rows in the key-run format (row t = the
 *                              page's token t);
 *   key meta    at kmeta_off:  the (scale, zero) pairs of the PT/group key
 *                              groups, key-run meta format;
 *   value codes at vcodes_off: PT/2 token-pair blocks, value-run format;
 *   value meta  at vmeta_off:  value-run meta format.
 * So a page block is exactly a key run and a value run of PT tokens:
 * kvq_quantize_append with codes = page + h0*head_bytes (+ the offset),
 * codes_stream_stride = meta_stream_stride = head_bytes and n_streams = the
 * sequence's kv heads writes the tokens of one page (dst_tok = token - j*PT).
 *   out[0] = head_bytes, out[1] = kmeta_off, out[2] = vcodes_off,
 *   out[3] = vmeta_off, out[4] = page_bytes = n_kv_heads * head_bytes
 *   (all multiples of 16).
 * page_tokens: a positive multiple of 64 and of group, at most 65536.
 * bits 2, 4 or 8; group in {32, 64, 128}, group <= d_h; d_h 64 or 128.
 */
kvq_status kvq_page_layout(int32_t n_kv_heads, int32_t d_h, int32_t group, int32_t bits,
                           int32_t page_tokens, int64_t out[5]);

typedef struct kvq_paged_args {
  int32_t batch, n_q_heads, n_kv_heads, d_h, group, bits;
  float sm_scale;             /* logit scale (1/sqrt(d_h) in the workloads)          */
  int32_t page_tokens;        /* PT, as in kvq_page_layout                           */
  const void* q;              /* fp16 [batch][n_q_heads][d_h]                        */
  const void* pages;          /* device pool; page p starts at pages + p*page_bytes  */
  int64_t page_bytes;         /* >= kvq_page_layout's page_bytes, multiple of 16     */
  const int32_t* block_table; /* device int32 [batch][max_pages]: sequence b's page j
                                 (its tokens j*PT .. j*PT+PT-1) is pool page
                                 block_table[b*max_pages + j]; the first
                                 ceil(n_kq/PT) entries of a row must address pages
                                 inside the pool (not checked on the device)      */
  int32_t max_pages;
  const int32_t* lengths;     /* host int32 [batch][4]: n_kq, n_vq, n_k_res, n_v_res */
  const int32_t* lengths_dev; /* device int32 [batch][4] holding the same values     */
  const void* k_res;          /* fp16 key residual: stream s = b*n_kv_heads + h has
                                 rows at element s*k_res_stride, row i = token n_kq + i */
  int64_t k_res_stride;
  const void* v_res;          /* fp16 value residual, row i = token n_vq + i         */
  int64_t v_res_stride;
  float* out;                 /* fp32 [batch][n_q_heads][d_h]                         */
  void* workspace;            /* device scratch, see kvq_decode_attn_paged_workspace  */
  size_t workspace_bytes;
} kvq_paged_args;

/*
 * Bytes of workspace kvq_decode_attn_paged needs (0 when every stream fits
 * one workgroup; then workspace may be NULL).  It depends on the shapes and
 * the host lengths only.  Partial softmax states; no initialization needed.
 */
kvq_status kvq_decode_attn_paged_workspace(const kvq_paged_args* args, size_t* bytes);

/*
 * kvq_decode_attn_paged -- decode attention over a paged, ragged cache: for
 * every (b, hq), with kv = hq / (n_q_heads / n_kv_heads), one softmax over
 * the sequence's N_b = n_kq + n_k_res logits (tokens 0..n_kq-1 dequantized
 * from its pages, then its key residual rows) and
 * out = sum_t p_t V'_t with tokens 0..n_vq-1 dequantized from the pages and
 * the rest from its value residual rows -- the same result as
 * kvq_decode_attn over one key run of n_kq and one value run of n_vq tokens.
 * Checks (all before any launch), per sequence: n_kq % group == 0,
 * 0 <= n_vq <= n_kq, n_k_res, n_v_res >= 0, n_kq + n_k_res == n_vq + n_v_res
 * = N_b with 1 <= N_b <= 2^22, ceil(n_kq / PT) <= max_pages; a value count
 * n_vq that is odd needs the missing pair partner's (scale, zero) finite
 * (kvq_quantize_append leaves it zero); pointers 16-byte aligned, residual
 * strides multiples of 8 elements, workspace large enough.  Reads the pages, the residuals and q; writes out and the
 * workspace only.
 */
kvq_status kvq_decode_attn_paged(const kvq_paged_args* args, void* stream);

/*
 * kvq_pq_search -- PQCache's decode-time PQ search (PQCache note,
 * "Background" on product quantization; "Method details", Steps 2 and 4):
 * for every batch row b and query head hq, with kv = hq / (n_q_heads /
 * n_kv_heads):
 *   table[j][c] = q[b][hq][j*dm .. j*dm+dm) . centroids[b][kv][j][c][0..dm)
 *                 for sub-space j < m, centroid c < 2^bits, dm = d_h / m
 *                 (fp32 sums of fp16 products);
 *   scores[b][hq][t] = sum_j table[j][codes[b][kv][t][j]]   (fp32, t < n_tok):
 *                 the query's dot product with the key rebuilt from the
 *                 centroids the token's codes name;
 *   top_idx[b][hq][0..top_k) = the top_k tokens with the largest scores,
 *                 ties to the lower token index, in ascending token order.
 * Layouts: q fp16 [batch][n_q_heads][d_h]; centroids fp16
 * [batch][n_kv_heads][m][2^bits][dm]; codes u8, stream s = b*n_kv_heads + kv
 * at codes + s*codes_stride bytes, [n_tok][m], each code < 2^bits (only its
 * low `bits` bits are read); scores fp32 [batch][n_q_heads][n_tok] (written);
 * top_idx int32 [batch][n_q_heads][top_k].
 * Two paths, one result: when a head's n_tok scores fit in a workgroup's LDS
 * (up to about 38K tokens) one kernel does all three steps per query head
 * with the scores resident in LDS; longer contexts run a scores kernel per
 * kv head (its query heads' tables in LDS) and a Top-k kernel that reads the
 * scores back.
 * Checks (before any launch): d_h 64 or 128; m divides 16 and d_h with dm a
 * multiple of 8; 1 <= bits <= 8; 1 <= top_k <= n_tok <= 2^24; codes_stride >= n_tok*m and a multiple of 16 (the kernel
 * reads up to the next multiple of 16 past n_tok*m); on the two-kernel path
 * the tables of a kv head's query heads (up to 8 at a time) fit 64 KB of LDS (KVQ_EUNSUPPORTED
 * otherwise); q, centroids, codes, scores 16-byte aligned, top_idx 4-byte
 * aligned.  Centroids and codes are inputs (the K-means construction of
 * Step 2 runs elsewhere).
 */
kvq_status kvq_pq_search(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t d_h,
                         int32_t m, int32_t bits, int32_t n_tok, int32_t top_k,
                         const void* q, const void* centroids, const void* codes,
                         int64_t codes_stride, float* scores, int32_t* top_idx, void* stream);

/*
 * kvq_vq_decode_attn -- decode attention over a vector-quantized (codebook)
 * KV cache (VQ-LLM note, "Background" on vector quantization and its CQ-2 /
 * CQ-4 KV-cache configurations): the key (value) of token t in kv head kv is,
 * in channels 4g .. 4g+3, the sum over rounds r < rounds of the codebook
 * entry k_books[kv][r][g][code] with code = k_codes[t][r][g] (likewise for
 * values); rounds = 1 is CQ-2 (2 bits per channel), rounds = 2 is CQ-4 (the
 * second round codes the residual of the first, 4 bits per channel).  For
 * every batch row b and query head hq, with kv = hq / (n_q_heads /
 * n_kv_heads):
 *   out[b][hq] = sum_t softmax_t(sm_scale * q[b][hq] . key_t) * value_t
 * over the n_tok cached tokens (fp32 accumulation).
 * Layouts: q fp16 [batch][n_q_heads][d_h]; k_codes, v_codes u8, stream
 * s = b*n_kv_heads + kv at codes + s*codes_stride bytes, [n_tok][rounds][d_h/4];
 * k_books, v_books fp16 [n_kv_heads][rounds][d_h/4][256][4] (shared by every
 * batch row); out fp32 [batch][n_q_heads][d_h].
 * workspace: device scratch of kvq_vq_decode_attn_workspace bytes (partial
 * softmax states of token chunks; 0 bytes, and NULL allowed, when each
 * stream is one chunk); calls sharing one must not overlap.
 * Checks (before any launch): d_h 64 or 128 (KVQ_EUNSUPPORTED); rounds 1 or
 * 2 (KVQ_EUNSUPPORTED); 1 <= n_tok <= 2^24 (at most 1024 chunks of up to
 * 8192 tokens); n_q_heads a multiple of n_kv_heads; codes_stride >=
 * n_tok*rounds*d_h/4 and a multiple of 16; q, codes and codebooks 16-byte
 * aligned, out 4-byte aligned; sm_scale finite.  Codebooks and codes are
 * inputs (their training runs elsewhere).  The value weights are summed with
 * LDS atomics, so the last bits of out may differ between runs.
 */
kvq_status kvq_vq_decode_attn_workspace(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                        int32_t d_h, int32_t rounds, int32_t n_tok, size_t* bytes);
kvq_status kvq_vq_decode_attn(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t d_h,
                              int32_t rounds, int32_t n_tok, float sm_scale, const void* q,
                              const void* k_codes, const void* v_codes, int64_t codes_stride,
                              const void* k_books, const void* v_books, float* out,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvq_window_thresholds -- the two score thresholds of a layer (WindowQuant
 * Sec. 3.2.3, Eq. 10 and 11): with s the layer's hidden-state similarity
 * (Eq. 9) and alpha the hyper-parameter,
 *   t_low  = (exp(alpha * s) - 1) / (exp(alpha) - 1),
 *   t_high = (exp(-alpha * s) - 1) / (exp(-alpha) - 1).
 * Host arithmetic in double, rounded to float.  alpha must be finite and
 * non-zero, s finite; KVQ_EINVAL otherwise.
 */
kvq_status kvq_window_thresholds(float layer_similarity, float alpha, float* t_low,
                                 float* t_high);

/*
 * kvq_window_search -- WindowQuant window-level quantization search (Sec.
 * 3.2) on the device: for batch row b and visual window i (visual tokens
 * i*S .. i*S+S-1; the floor(n_visual/S) full windows, trailing tokens are no
 * window), the score is the mean cosine similarity over all pairs of a text
 * token and a token of the window (Eq. 8); the row's choice is fp16 (16) for
 * score > t_high, int2 (2) for score < t_low, int4 (4) otherwise (Sec.
 * 3.2.1); the window's width is the choice most rows made, ties to the wider
 * width (Sec. 3.2.3); with first_window_fp16, window 0 is 16 regardless
 * (Sec. 3.2.2).  A token row of zero length counts as cosine 0 with every
 * other token.  Scores are computed in fp32 (the mean of unit vectors' dot
 * products as the dot product of their sums).
 *   text     fp16 rows, row j of batch row b at element
 *            b*text_batch_stride + j*text_row_stride; likewise visual.
 *   dim      D, a multiple of 8, 8..4096.  n_text, window_tokens >= 1;
 *            n_visual >= window_tokens.
 *   scores   NULL or device float [batch][n_visual / window_tokens].
 *   win_bits device uint8 [n_visual / window_tokens] (input of
 *            kvq_reorder_windows).
 *   workspace  device scratch of kvq_window_search_workspace bytes (chunk
 *            sums; no initialization needed; calls sharing one must not
 *            overlap).
 * Pointers 16-byte aligned (scores 4), strides multiples of 8 elements and
 * row strides >= dim.
 */
kvq_status kvq_window_search_workspace(int32_t batch, int32_t n_text, int32_t n_visual,
                                       int32_t dim, int32_t window_tokens, size_t* bytes);
kvq_status kvq_window_search(int32_t batch, int32_t n_text, int32_t n_visual, int32_t dim,
                             const void* text, int64_t text_batch_stride,
                             int64_t text_row_stride, const void* visual,
                             int64_t visual_batch_stride, int64_t visual_row_stride,
                             int32_t window_tokens, float t_low, float t_high,
                             int32_t first_window_fp16, float* scores, uint8_t* win_bits,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * A KIVI cache of n_streams = B * Hkv streams in the state that KIVI's
 * Algorithm 1 keeps between decode steps: one key run and one value run of
 * b-bit codes (code and meta arenas with code_off = meta_off = 0, room for
 * `capacity` tokens each), the fp16 key residual (R rows per stream) and the
 * fp16 value window (a ring of win_rows rows per stream; the window's r_v
 * rows start at row v_start).  The caller allocates every buffer; the five
 * lengths are host integers that kvq_kivi_step reads and updates.
 */
typedef struct kvq_kivi_cache {
  int32_t bits;           /* 2, 4 or 8                                         */
  int32_t group;          /* G in {32, 64, 128}, G <= d_h                      */
  int32_t residual;       /* R, a positive multiple of G                       */
  int32_t n_streams;      /* B * Hkv >= 1                                      */
  int32_t d_h;            /* 64 or 128                                         */
  int32_t capacity;       /* tokens the key and value runs have room for       */
  int32_t win_rows;       /* value-window rows per stream, >= 2R + 2           */
  int32_t reserved;       /* must be 0                                         */
  void* k_codes;  int64_t k_codes_stride;   /* arenas: base, bytes per stream */
  void* k_meta;   int64_t k_meta_stride;
  void* v_codes;  int64_t v_codes_stride;
  void* v_meta;   int64_t v_meta_stride;
  void* k_res;    int64_t k_res_stride;     /* fp16 elements per stream         */
  void* v_res;    int64_t v_res_stride;
  /* state: tokens in the key run, key residual, value run, value window,
   * and the window's first row (n_kq + r_k == n_vq + r_v) */
  int32_t n_kq, r_k, n_vq, r_v, v_start;
  /* out: kernel launches the last kvq_kivi_step enqueued (1 when the append
   * ran fused into the attention kernel) */
  int32_t last_launches;
} kvq_kivi_cache;

/*
 * Workspace bytes kvq_kivi_step needs for its attention call with the cache
 * in the state the step leaves it in (see kvq_decode_attn_workspace).
 */
kvq_status kvq_kivi_step_workspace(const kvq_kivi_cache* cache, int32_t batch,
                                   int32_t n_q_heads, size_t* bytes);

/*
 * kvq_kivi_step -- one whole KIVI decode step in one call (Algorithm 1,
 * Decoding, followed by the attention of the new token's queries):
 *   1. when the window ring has no free row after its last one, the r_v
 *      window rows move to rows 0..r_v-1 (v_start = 0);
 *   2. the new key row becomes key-residual row r_k and the new value row
 *      window row v_start + r_v; if the window then holds more than R
 *      values, its oldest one is quantized per token and appended to the
 *      value run (kvq_decode_append);
 *   3. if the key residual now holds R rows, they are quantized as R/G whole
 *      groups and appended to the key run (kvq_quantize_append), r_k = 0;
 *   4. kvq_decode_attn of q over the updated cache (split chosen by the
 *      library) writes out.
 * When no compaction and no key flush is due, each stream fits one workgroup
 * per head block (of up to 4 query heads) and every token the append writes
 * falls in the range of that workgroup's last wave, steps 2 and 4 run as one
 * launch: that wave performs the stream's append first, with the same
 * arithmetic, so the result is the same as the separate calls (with several
 * head blocks each block's last wave writes the same bytes).
 *   k_new, v_new  fp16 rows, stream s at element s * new_stride.
 *   q, out        fp16 [batch][n_q_heads][d_h] and fp32 [batch][n_q_heads][d_h];
 *                 n_streams = batch * n_kv_heads with n_kv_heads dividing
 *                 n_q_heads.
 * All checks (shapes, state consistency, capacity, workspace) run before
 * anything is enqueued; on success the five lengths in *cache are updated.
 * On KVQ_ELAUNCH the cache contents and lengths are undefined.
 */
kvq_status kvq_kivi_step(kvq_kivi_cache* cache, int32_t batch, int32_t n_q_heads,
                         float sm_scale, const void* k_new, int64_t k_new_stride,
                         const void* v_new, int64_t v_new_stride, const void* q,
                         float* out, void* workspace, size_t workspace_bytes,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
