"""kvq -- decode attention over a low-bit quantized KV cache on MI355X (gfx950).

Python binding of the C ABI in ``include/kvq.h``.  Every function here has
the name and argument list of the C entry point; the binding only turns torch
tensors into device pointers, picks torch's current HIP stream when none is
given, and raises :class:`KvqError` on a non-zero status.  All computation
happens in the HIP kernels of ``libkvq.so``; there is no fallback: if the
library is missing, importing a function that needs it raises.

``decode_attention_kivi_amd.cache`` holds the cache bookkeeping (KIVI's
residual / flush rules and the WindowQuant reorder flow) built on these calls.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

__all__ = [
    "KVQ_KEYS", "KVQ_VALUES", "KvqError", "Segment", "DecodeArgs", "library_path",
    "kvq_abi_version", "kvq_strerror", "kvq_quantize_append", "kvq_residual_append",
    "kvq_decode_append",
    "kvq_reorder_windows", "kvq_decode_attn_workspace", "kvq_decode_attn", "kvq_decode_attn_noalloc",
    "KVQ_SCRATCH_BYTES",
    "KiviCacheDesc", "kvq_kivi_step_workspace", "kvq_kivi_step",
    "kvq_window_thresholds", "kvq_window_search_workspace", "kvq_window_search",
    "PagedArgs", "kvq_page_layout", "kvq_decode_attn_paged_workspace", "kvq_decode_attn_paged",
    "kvq_pq_search", "kvq_vq_decode_attn_workspace", "kvq_vq_decode_attn",
]

KVQ_KEYS = 0
KVQ_VALUES = 1
KVQ_SCRATCH_BYTES = 8 << 20     # the library's static scratch (kvq_decode_attn_noalloc)
ABI_VERSION = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIBRARY names another library file in this directory (a comparison
# build of build.VARIANTS); by default libkvq.so
_LIB_PATH = os.path.join(_HERE, os.path.basename(os.environ.get("KVQ_LIBRARY") or "libkvq.so"))
_lib = None


class KvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {kvq_strerror(status)} (status {status})")


class Segment(ctypes.Structure):
    """kvq_segment: one run of consecutive cache tokens at one bit width."""
    _fields_ = [("bits", ctypes.c_int32), ("tok_begin", ctypes.c_int32),
                ("n_tok", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("code_off", ctypes.c_int64), ("meta_off", ctypes.c_int64)]

    def astuple(self):
        return (self.bits, self.tok_begin, self.n_tok, self.code_off, self.meta_off)


class DecodeArgs(ctypes.Structure):
    """kvq_decode_args (field order and types of include/kvq.h)."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("d_h", ctypes.c_int32),
        ("group", ctypes.c_int32), ("sm_scale", ctypes.c_float),
        ("q", ctypes.c_void_p),
        ("k_segs", ctypes.POINTER(Segment)), ("n_k_segs", ctypes.c_int32),
        ("v_segs", ctypes.POINTER(Segment)), ("n_v_segs", ctypes.c_int32),
        ("k_codes", ctypes.c_void_p), ("k_codes_stride", ctypes.c_int64),
        ("k_meta", ctypes.c_void_p), ("k_meta_stride", ctypes.c_int64),
        ("v_codes", ctypes.c_void_p), ("v_codes_stride", ctypes.c_int64),
        ("v_meta", ctypes.c_void_p), ("v_meta_stride", ctypes.c_int64),
        ("k_res", ctypes.c_void_p), ("n_k_res", ctypes.c_int32), ("k_res_stride", ctypes.c_int64),
        ("v_res", ctypes.c_void_p), ("n_v_res", ctypes.c_int32), ("v_res_stride", ctypes.c_int64),
        ("out", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("split_tokens", ctypes.c_int32),
    ]


class KiviCacheDesc(ctypes.Structure):
    """kvq_kivi_cache (field order and types of include/kvq.h)."""
    _fields_ = [
        ("bits", ctypes.c_int32), ("group", ctypes.c_int32), ("residual", ctypes.c_int32),
        ("n_streams", ctypes.c_int32), ("d_h", ctypes.c_int32), ("capacity", ctypes.c_int32),
        ("win_rows", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("k_codes", ctypes.c_void_p), ("k_codes_stride", ctypes.c_int64),
        ("k_meta", ctypes.c_void_p), ("k_meta_stride", ctypes.c_int64),
        ("v_codes", ctypes.c_void_p), ("v_codes_stride", ctypes.c_int64),
        ("v_meta", ctypes.c_void_p), ("v_meta_stride", ctypes.c_int64),
        ("k_res", ctypes.c_void_p), ("k_res_stride", ctypes.c_int64),
        ("v_res", ctypes.c_void_p), ("v_res_stride", ctypes.c_int64),
        ("n_kq", ctypes.c_int32), ("r_k", ctypes.c_int32), ("n_vq", ctypes.c_int32),
        ("r_v", ctypes.c_int32), ("v_start", ctypes.c_int32), ("last_launches", ctypes.c_int32),
    ]


class PagedArgs(ctypes.Structure):
    """kvq_paged_args (field order and types of include/kvq.h)."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("d_h", ctypes.c_int32), ("group", ctypes.c_int32), ("bits", ctypes.c_int32),
        ("sm_scale", ctypes.c_float), ("page_tokens", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("pages", ctypes.c_void_p), ("page_bytes", ctypes.c_int64),
        ("block_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32),
        ("lengths", ctypes.c_void_p), ("lengths_dev", ctypes.c_void_p),
        ("k_res", ctypes.c_void_p), ("k_res_stride", ctypes.c_int64),
        ("v_res", ctypes.c_void_p), ("v_res_stride", ctypes.c_int64),
        ("out", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                          "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(_LIB_PATH)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.kvq_abi_version.restype = i32
    lib.kvq_abi_version.argtypes = []
    lib.kvq_strerror.restype = ctypes.c_char_p
    lib.kvq_strerror.argtypes = [i32]
    lib.kvq_quantize_append.restype = i32
    lib.kvq_quantize_append.argtypes = [i32, i32, i32, i32, i32, i32, vp, i64, i64, vp,
                                        vp, i64, vp, i64, i32, vp]
    lib.kvq_residual_append.restype = i32
    lib.kvq_residual_append.argtypes = [i32, i32, i32, vp, i64, i64, vp, i64, i32, vp]
    lib.kvq_decode_append.restype = i32
    lib.kvq_decode_append.argtypes = [i32, i32, i32, i32, vp, i64, vp, i64, vp, i64, i32,
                                      vp, i64, i32, i32, vp, i64, vp, i64, i32, vp]
    lib.kvq_reorder_windows.restype = i32
    lib.kvq_reorder_windows.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp]
    lib.kvq_decode_attn_workspace.restype = i32
    lib.kvq_decode_attn_workspace.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.POINTER(ctypes.c_size_t)]
    lib.kvq_decode_attn.restype = i32
    lib.kvq_decode_attn.argtypes = [ctypes.POINTER(DecodeArgs), vp]
    lib.kvq_decode_attn_noalloc.restype = i32
    lib.kvq_decode_attn_noalloc.argtypes = [ctypes.POINTER(DecodeArgs), vp]
    lib.kvq_kivi_step_workspace.restype = i32
    lib.kvq_kivi_step_workspace.argtypes = [ctypes.POINTER(KiviCacheDesc), i32, i32,
                                            ctypes.POINTER(ctypes.c_size_t)]
    lib.kvq_window_thresholds.restype = i32
    lib.kvq_window_thresholds.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.POINTER(ctypes.c_float),
                                          ctypes.POINTER(ctypes.c_float)]
    lib.kvq_window_search_workspace.restype = i32
    lib.kvq_window_search_workspace.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.kvq_window_search.restype = i32
    lib.kvq_window_search.argtypes = [i32, i32, i32, i32, vp, i64, i64, vp, i64, i64, i32,
                                      ctypes.c_float, ctypes.c_float, i32, vp, vp, vp, ctypes.c_size_t, vp]
    lib.kvq_kivi_step.restype = i32
    lib.kvq_kivi_step.argtypes = [ctypes.POINTER(KiviCacheDesc), i32, i32, ctypes.c_float,
                                  vp, i64, vp, i64, vp, vp, vp, ctypes.c_size_t, vp]
    lib.kvq_page_layout.restype = i32
    lib.kvq_page_layout.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_int64)]
    lib.kvq_decode_attn_paged_workspace.restype = i32
    lib.kvq_decode_attn_paged_workspace.argtypes = [ctypes.POINTER(PagedArgs), ctypes.POINTER(ctypes.c_size_t)]
    lib.kvq_decode_attn_paged.restype = i32
    lib.kvq_decode_attn_paged.argtypes = [ctypes.POINTER(PagedArgs), vp]
    lib.kvq_pq_search.restype = i32
    lib.kvq_pq_search.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, i64, vp, vp, vp]
    lib.kvq_vq_decode_attn_workspace.restype = i32
    lib.kvq_vq_decode_attn_workspace.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.kvq_vq_decode_attn.restype = i32
    lib.kvq_vq_decode_attn.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.c_float, vp, vp, vp, i64,
                                       vp, vp, vp, vp, ctypes.c_size_t, vp]
    if lib.kvq_abi_version() != ABI_VERSION:
        raise ImportError(f"libkvq ABI {lib.kvq_abi_version()} != binding ABI {ABI_VERSION}")
    _lib = lib
    return lib


def _dev(x) -> Optional[int]:
    """Device pointer of a CUDA tensor (None -> NULL); ints pass through."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not getattr(x, "is_cuda", False):
        raise ValueError("device buffer expected (a CUDA tensor or an int address)")
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != 0:
        raise KvqError(status, where)


def kvq_abi_version() -> int:
    return int(_load().kvq_abi_version())


def kvq_strerror(status: int) -> str:
    return _load().kvq_strerror(int(status)).decode()


def kvq_quantize_append(which, bits, group, n_streams, d_h, n_tok, src, src_stream_stride,
                        src_row_stride, src_rows, codes, codes_stream_stride, meta,
                        meta_stream_stride, dst_tok, stream=None):
    """See include/kvq.h.  Strides: src in fp16 elements, codes/meta in bytes."""
    _check(_load().kvq_quantize_append(
        which, bits, group, n_streams, d_h, n_tok, _dev(src), src_stream_stride, src_row_stride,
        _dev(src_rows), _dev(codes), codes_stream_stride, _dev(meta), meta_stream_stride,
        dst_tok, _stream(stream)), "kvq_quantize_append")


def kvq_residual_append(n_streams, d_h, n_rows, src, src_stream_stride, src_row_stride, dst,
                        dst_stream_stride, dst_row, stream=None):
    """See include/kvq.h.  Strides in fp16 elements."""
    _check(_load().kvq_residual_append(
        n_streams, d_h, n_rows, _dev(src), src_stream_stride, src_row_stride, _dev(dst),
        dst_stream_stride, dst_row, _stream(stream)), "kvq_residual_append")


def kvq_decode_append(bits, group, n_streams, d_h, k_new, k_new_stride, v_new, v_new_stride,
                      k_res, k_res_stride, k_row, v_res, v_res_stride, v_row, v_quant_row,
                      v_codes, v_codes_stride, v_meta, v_meta_stride, v_dst_tok, stream=None):
    """See include/kvq.h.  Row strides in fp16 elements, code/meta strides in bytes."""
    _check(_load().kvq_decode_append(
        bits, group, n_streams, d_h, _dev(k_new), k_new_stride, _dev(v_new), v_new_stride,
        _dev(k_res), k_res_stride, k_row, _dev(v_res), v_res_stride, v_row, v_quant_row,
        _dev(v_codes), v_codes_stride, _dev(v_meta), v_meta_stride, v_dst_tok, _stream(stream)),
        "kvq_decode_append")


def kvq_reorder_windows(win_bits, n_windows, window_tokens, group, d_h, perm, segs, n_segs,
                        row_gather, stream=None):
    """See include/kvq.h.  ``segs`` is a device buffer of 4 kvq_segment (128 bytes)."""
    _check(_load().kvq_reorder_windows(
        _dev(win_bits), n_windows, window_tokens, group, d_h, _dev(perm), _dev(segs),
        _dev(n_segs), _dev(row_gather), _stream(stream)), "kvq_reorder_windows")


def segments(rows: Sequence) -> ctypes.Array:
    """Host kvq_segment array from (bits, tok_begin, n_tok, code_off, meta_off) rows."""
    arr = (Segment * max(1, len(rows)))()
    for i, r in enumerate(rows):
        arr[i] = Segment(int(r[0]), int(r[1]), int(r[2]), 0, int(r[3]), int(r[4]))
    return arr


def make_decode_args(*, batch, n_q_heads, n_kv_heads, d_h, group, sm_scale, q,
                     k_segs=(), v_segs=(), k_codes=None, k_codes_stride=0, k_meta=None,
                     k_meta_stride=0, v_codes=None, v_codes_stride=0, v_meta=None,
                     v_meta_stride=0, k_res=None, n_k_res=0, k_res_stride=0, v_res=None,
                     n_v_res=0, v_res_stride=0, out=None, workspace=None, workspace_bytes=0,
                     split_tokens=0) -> DecodeArgs:
    """Fill a kvq_decode_args; segments are (bits, tok_begin, n_tok, code_off, meta_off)."""
    ks, vs = segments(k_segs), segments(v_segs)
    a = DecodeArgs(
        batch, n_q_heads, n_kv_heads, d_h, group, float(sm_scale), _dev(q),
        ks, len(k_segs), vs, len(v_segs),
        _dev(k_codes), k_codes_stride, _dev(k_meta), k_meta_stride,
        _dev(v_codes), v_codes_stride, _dev(v_meta), v_meta_stride,
        _dev(k_res), n_k_res, k_res_stride, _dev(v_res), n_v_res, v_res_stride,
        _dev(out), _dev(workspace), int(workspace_bytes), int(split_tokens))
    a._keep = (ks, vs)          # the segment arrays must outlive the call
    return a


def kvq_decode_attn_workspace(args: DecodeArgs) -> int:
    n = ctypes.c_size_t(0)
    _check(_load().kvq_decode_attn_workspace(ctypes.byref(args), ctypes.byref(n)),
           "kvq_decode_attn_workspace")
    return int(n.value)


def kvq_decode_attn(args: DecodeArgs, stream=None):
    _check(_load().kvq_decode_attn(ctypes.byref(args), _stream(stream)), "kvq_decode_attn")


def kvq_decode_attn_noalloc(args: DecodeArgs, stream=None):
    """kvq_decode_attn with the partial states in the library's static scratch
    (``args.workspace`` is ignored); for callers that cannot allocate."""
    _check(_load().kvq_decode_attn_noalloc(ctypes.byref(args), _stream(stream)), "kvq_decode_attn_noalloc")


def kvq_kivi_step_workspace(cache: KiviCacheDesc, batch: int, n_q_heads: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_load().kvq_kivi_step_workspace(ctypes.byref(cache), batch, n_q_heads, ctypes.byref(n)),
           "kvq_kivi_step_workspace")
    return int(n.value)


def kvq_kivi_step(cache: KiviCacheDesc, batch, n_q_heads, sm_scale, k_new, k_new_stride, v_new,
                  v_new_stride, q, out, workspace=None, workspace_bytes=0, stream=None):
    """One KIVI decode step; updates the lengths in ``cache`` (a KiviCacheDesc)."""
    _check(_load().kvq_kivi_step(ctypes.byref(cache), batch, n_q_heads, float(sm_scale),
                                 _dev(k_new), k_new_stride, _dev(v_new), v_new_stride, _dev(q),
                                 _dev(out), _dev(workspace), int(workspace_bytes), _stream(stream)),
           "kvq_kivi_step")


def kvq_window_thresholds(layer_similarity: float, alpha: float):
    """(t_low, t_high) of a layer, WindowQuant Eq. 10-11."""
    lo, hi = ctypes.c_float(0), ctypes.c_float(0)
    _check(_load().kvq_window_thresholds(float(layer_similarity), float(alpha), ctypes.byref(lo),
                                         ctypes.byref(hi)), "kvq_window_thresholds")
    return float(lo.value), float(hi.value)


def kvq_window_search_workspace(batch, n_text, n_visual, dim, window_tokens) -> int:
    n = ctypes.c_size_t(0)
    _check(_load().kvq_window_search_workspace(batch, n_text, n_visual, dim, window_tokens, ctypes.byref(n)),
           "kvq_window_search_workspace")
    return int(n.value)


def kvq_window_search(batch, n_text, n_visual, dim, text, text_batch_stride, text_row_stride, visual,
                      visual_batch_stride, visual_row_stride, window_tokens, t_low, t_high,
                      first_window_fp16, scores, win_bits, workspace, workspace_bytes, stream=None):
    _check(_load().kvq_window_search(batch, n_text, n_visual, dim, _dev(text), text_batch_stride,
                                     text_row_stride, _dev(visual), visual_batch_stride, visual_row_stride,
                                     window_tokens, float(t_low), float(t_high), int(first_window_fp16),
                                     _dev(scores), _dev(win_bits), _dev(workspace), int(workspace_bytes),
                                     _stream(stream)), "kvq_window_search")


def kvq_page_layout(n_kv_heads, d_h, group, bits, page_tokens) -> dict:
    """Byte layout of one page of the paged cache (head_bytes, kmeta_off,
    vcodes_off, vmeta_off, page_bytes)."""
    out = (ctypes.c_int64 * 5)()
    _check(_load().kvq_page_layout(n_kv_heads, d_h, group, bits, page_tokens, out), "kvq_page_layout")
    return dict(zip(("head_bytes", "kmeta_off", "vcodes_off", "vmeta_off", "page_bytes"), (int(x) for x in out)))


def kvq_decode_attn_paged_workspace(args: PagedArgs) -> int:
    n = ctypes.c_size_t(0)
    _check(_load().kvq_decode_attn_paged_workspace(ctypes.byref(args), ctypes.byref(n)),
           "kvq_decode_attn_paged_workspace")
    return int(n.value)


def kvq_decode_attn_paged(args: PagedArgs, stream=None):
    _check(_load().kvq_decode_attn_paged(ctypes.byref(args), _stream(stream)), "kvq_decode_attn_paged")


def kvq_pq_search(batch, n_q_heads, n_kv_heads, d_h, m, bits, n_tok, top_k, q, centroids, codes,
                  codes_stride, scores, top_idx, stream=None):
    """PQCache decode-time PQ search: approximate scores and Top-k tokens."""
    _check(_load().kvq_pq_search(batch, n_q_heads, n_kv_heads, d_h, m, bits, n_tok, top_k, _dev(q),
                                 _dev(centroids), _dev(codes), int(codes_stride), _dev(scores),
                                 _dev(top_idx), _stream(stream)), "kvq_pq_search")


def kvq_vq_decode_attn_workspace(batch, n_q_heads, n_kv_heads, d_h, rounds, n_tok) -> int:
    n = ctypes.c_size_t(0)
    _check(_load().kvq_vq_decode_attn_workspace(batch, n_q_heads, n_kv_heads, d_h, rounds, n_tok, ctypes.byref(n)),
           "kvq_vq_decode_attn_workspace")
    return int(n.value)


def kvq_vq_decode_attn(batch, n_q_heads, n_kv_heads, d_h, rounds, n_tok, sm_scale, q, k_codes, v_codes,
                       codes_stride, k_books, v_books, out, workspace=None, workspace_bytes=0, stream=None):
    """Decode attention over a vector-quantized (codebook) KV cache."""
    _check(_load().kvq_vq_decode_attn(batch, n_q_heads, n_kv_heads, d_h, rounds, n_tok, float(sm_scale), _dev(q),
                                      _dev(k_codes), _dev(v_codes), int(codes_stride), _dev(k_books),
                                      _dev(v_books), _dev(out), _dev(workspace), int(workspace_bytes),
                                      _stream(stream)), "kvq_vq_decode_attn")
