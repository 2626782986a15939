"""Cache bookkeeping on top of the kvq C ABI.

``KiviCache`` keeps the KIVI cache of a batch: quantized keys and values in
device arenas, an fp16 key residual and an fp16 value window, and the host
integers that say how many tokens each part holds.  It follows the KIVI
note's Algorithm 1: prefill quantizes values up to l - R and keys up to
l - l%R; each decode step appends the new token's key and value to the
residuals, flushes the key residual as a whole when it reaches R tokens and
quantizes the oldest values beyond R.  The attention call then reads
[quantized keys | key residual] and [quantized values | value window].

``PagedKiviCache`` keeps the same KIVI state per sequence with its own
lengths (a ragged batch), the quantized tokens in fixed-size pages of a
shared pool listed by a block table (the serving layout the KIVI note's
outlook pairs with PagedAttention).

``WindowCache`` keeps a WindowQuant cache (Sec. 3.1, 3.3.1): the visual
windows are reordered by bit width on the device, each run is quantized from
the gathered rows, and the text/new tokens stay fp16.

All data movement and arithmetic runs in libkvq's kernels; this module only
allocates device buffers (torch) and tracks lengths.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

from . import (KVQ_KEYS, KVQ_VALUES, KiviCacheDesc, PagedArgs, Segment, kvq_decode_append,
               kvq_decode_attn, kvq_decode_attn_paged, kvq_decode_attn_paged_workspace,
               kvq_decode_attn_workspace, kvq_kivi_step, kvq_kivi_step_workspace, kvq_page_layout,
               kvq_quantize_append, kvq_reorder_windows, kvq_residual_append, make_decode_args)

__all__ = ["KiviCache", "WindowCache", "PagedKiviCache", "arena_bytes", "kivi_step_lengths"]


def _round16(x: int) -> int:
    return (x + 15) // 16 * 16


def arena_bytes(bits: int, n_tok: int, d: int, group: int) -> Tuple[int, int, int, int]:
    """(key code, key meta, value code, value meta) bytes per stream for a run."""
    if bits == 16:
        return _round16(n_tok * d * 2), 0, _round16(n_tok * d * 2), 0
    k_codes = n_tok * d * bits // 8
    k_meta = (n_tok // group) * d * 4
    pairs = (n_tok + 1) // 2
    v_codes = pairs * d * bits // 4
    v_meta = pairs * (d // group) * 8
    return tuple(_round16(x) for x in (k_codes, k_meta, v_codes, v_meta))


def _streams(x: torch.Tensor) -> Tuple[int, int, int]:
    """(n_streams, stream stride, row stride) of a [B][H][N][d] fp16 view."""
    assert x.dtype == torch.float16 and x.is_cuda and x.dim() == 4 and x.stride(3) == 1
    b, h = x.shape[0], x.shape[1]
    if b > 1 and h > 1:
        assert x.stride(0) == h * x.stride(1), "batch and head dims must collapse"
    ss = x.stride(1) if h > 1 else x.stride(0)
    return b * h, ss, x.stride(2)


class KiviCache:
    """KIVI cache of B x Hkv streams with group G, residual R, ``bits``-bit codes."""

    def __init__(self, batch: int, n_kv_heads: int, d_h: int, bits: int, group: int,
                 residual: int, capacity: int, device="cuda"):
        assert residual % group == 0 and capacity >= 1
        self.B, self.H, self.d, self.bits, self.G, self.R = batch, n_kv_heads, d_h, bits, group, residual
        self.n_streams = batch * n_kv_heads
        cap = (capacity + group - 1) // group * group
        self.capacity = cap
        kc, km, vc, vm = arena_bytes(bits, cap, d_h, group)
        u8 = dict(dtype=torch.uint8, device=device)
        self.k_codes = torch.zeros(self.n_streams, kc, **u8)
        self.k_meta = torch.zeros(self.n_streams, km, **u8)
        self.v_codes = torch.zeros(self.n_streams, vc, **u8)
        self.v_meta = torch.zeros(self.n_streams, vm, **u8)
        f16 = dict(dtype=torch.float16, device=device)
        self.k_res = torch.zeros(self.n_streams, residual, d_h, **f16)
        # value window: rows [v_start, v_start + r_v); compacted to row 0 when full
        self.v_win_rows = 2 * residual + 2
        self.v_res = torch.zeros(self.n_streams, self.v_win_rows, d_h, **f16)
        self.n_kq = self.r_k = self.n_vq = self.r_v = self.v_start = 0
        self.last_launches = 0
        self._ws = None
        self._need = {}

    # -- state ---------------------------------------------------------------
    @property
    def lengths(self):
        return self.n_kq, self.r_k, self.n_vq, self.r_v

    @property
    def n_tokens(self) -> int:
        return self.n_kq + self.r_k

    def _quant(self, which, src_ptr_view: torch.Tensor, n_tok: int, ss: int, rs: int, dst_tok: int,
               stream=None):
        codes, meta = (self.k_codes, self.k_meta) if which == KVQ_KEYS else (self.v_codes, self.v_meta)
        kvq_quantize_append(which, self.bits, self.G, self.n_streams, self.d, n_tok, src_ptr_view,
                            ss, rs, None, codes, codes.stride(0), meta, meta.stride(0), dst_tok,
                            stream)

    def prefill(self, k: torch.Tensor, v: torch.Tensor, stream=None):
        """Quantize the prompt's keys/values [B][Hkv][l][d] (fp16, on the device)."""
        assert self.n_tokens == 0
        n, ss, rs = _streams(k)
        n2, ss2, rs2 = _streams(v)
        l = k.shape[2]
        assert n == self.n_streams and v.shape[2] == l and l <= self.capacity
        n_vq = max(l - self.R, 0)
        if n_vq:
            self._quant(KVQ_VALUES, v, n_vq, ss2, rs2, 0, stream)
        if l - n_vq:
            kvq_residual_append(n, self.d, l - n_vq, v[:, :, n_vq:], ss2, rs2, self.v_res,
                                self.v_res.stride(0), 0, stream)
        n_kq = l - l % self.R
        if n_kq:
            self._quant(KVQ_KEYS, k, n_kq, ss, rs, 0, stream)
        if l - n_kq:
            kvq_residual_append(n, self.d, l - n_kq, k[:, :, n_kq:], ss, rs, self.k_res,
                                self.k_res.stride(0), 0, stream)
        self.n_kq, self.r_k, self.n_vq, self.r_v, self.v_start = n_kq, l - n_kq, n_vq, l - n_vq, 0

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor, stream=None):
        """Decode-step append of one token per stream ([B][Hkv][1][d] fp16).

        One kvq_decode_append call writes the key residual row and the value
        window row and quantizes the oldest value beyond R; the rare key flush
        (every R steps) and window compaction are separate calls.
        """
        assert self.n_tokens + 1 <= self.capacity
        n, ss, _ = _streams(k_new)
        n2, ss2, _ = _streams(v_new)
        assert n == n2 == self.n_streams
        if self.v_start + self.r_v + 1 > self.v_win_rows:
            kvq_residual_append(n, self.d, self.r_v, self.v_res[:, self.v_start:], self.v_res.stride(0),
                                self.d, self.v_res, self.v_res.stride(0), 0, stream)
            self.v_start = 0
        v_row = self.v_start + self.r_v
        quant = self.r_v + 1 > self.R            # the window then holds R + 1 values
        kvq_decode_append(self.bits, self.G, n, self.d, k_new, ss, v_new, ss2,
                          self.k_res, self.k_res.stride(0), self.r_k,
                          self.v_res, self.v_res.stride(0), v_row,
                          self.v_start if quant else -1,
                          self.v_codes, self.v_codes.stride(0), self.v_meta, self.v_meta.stride(0),
                          self.n_vq, stream)
        self.r_k += 1
        self.r_v += 1
        if quant:
            self.n_vq += 1
            self.v_start += 1
            self.r_v -= 1
        # keys: flush R tokens as whole groups when the residual is full
        if self.r_k == self.R:
            self._quant(KVQ_KEYS, self.k_res.unsqueeze(1), self.R, self.k_res.stride(0), self.d,
                        self.n_kq, stream)
            self.n_kq += self.R
            self.r_k = 0

    def decode_args(self, q: torch.Tensor, out: torch.Tensor, sm_scale: float,
                    split_tokens: int = 0):
        B, Hq, d = q.shape
        assert B == self.B and d == self.d and q.is_contiguous() and q.dtype == torch.float16
        kseg = [(self.bits, 0, self.n_kq, 0, 0)] if self.n_kq else []
        vseg = [(self.bits, 0, self.n_vq, 0, 0)] if self.n_vq else []
        a = make_decode_args(
            batch=B, n_q_heads=Hq, n_kv_heads=self.H, d_h=d, group=self.G, sm_scale=sm_scale, q=q,
            k_segs=kseg, v_segs=vseg,
            k_codes=self.k_codes, k_codes_stride=self.k_codes.stride(0),
            k_meta=self.k_meta, k_meta_stride=self.k_meta.stride(0),
            v_codes=self.v_codes, v_codes_stride=self.v_codes.stride(0),
            v_meta=self.v_meta, v_meta_stride=self.v_meta.stride(0),
            k_res=self.k_res, n_k_res=self.r_k, k_res_stride=self.k_res.stride(0),
            v_res=self.v_res.data_ptr() + self.v_start * d * 2, n_v_res=self.r_v,
            v_res_stride=self.v_res.stride(0), out=out, split_tokens=split_tokens)
        # the workspace size depends on the shapes and lengths only: asked
        # once per state instead of planning twice per call
        key = (B, Hq, self.lengths, split_tokens)
        need = self._need.get(key)
        if need is None:
            need = self._need[key] = kvq_decode_attn_workspace(a)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        a.workspace = self._ws.data_ptr()
        a.workspace_bytes = self._ws.numel()
        return a

    def attend(self, q: torch.Tensor, sm_scale: float, out: Optional[torch.Tensor] = None,
               split_tokens: int = 0, stream=None) -> torch.Tensor:
        """Decode attention of q [B][Hq][d] (fp16) -> fp32 [B][Hq][d]."""
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        kvq_decode_attn(self.decode_args(q, out, sm_scale, split_tokens), stream)
        return out

    def desc(self) -> KiviCacheDesc:
        """The cache as the C ABI's kvq_kivi_cache (buffers and current lengths)."""
        return KiviCacheDesc(
            self.bits, self.G, self.R, self.n_streams, self.d, self.capacity, self.v_win_rows, 0,
            self.k_codes.data_ptr(), self.k_codes.stride(0), self.k_meta.data_ptr(), self.k_meta.stride(0),
            self.v_codes.data_ptr(), self.v_codes.stride(0), self.v_meta.data_ptr(), self.v_meta.stride(0),
            self.k_res.data_ptr(), self.k_res.stride(0), self.v_res.data_ptr(), self.v_res.stride(0),
            self.n_kq, self.r_k, self.n_vq, self.r_v, self.v_start, 0)

    def step(self, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor, sm_scale: float,
             out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """append() followed by attend(), as one kvq_kivi_step call."""
        assert self.n_tokens + 1 <= self.capacity
        n, ss, _ = _streams(k_new)
        n2, ss2, _ = _streams(v_new)
        B, Hq, d = q.shape
        assert n == n2 == self.n_streams and B == self.B and d == self.d
        assert q.is_contiguous() and q.dtype == torch.float16
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        c = self.desc()
        need = kvq_kivi_step_workspace(c, B, Hq)
        if need and (self._ws is None or self._ws.numel() < need):
            self._ws = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws = self._ws if need else None
        kvq_kivi_step(c, B, Hq, sm_scale, k_new, ss, v_new, ss2, q, out, ws,
                      ws.numel() if ws is not None else 0, stream)
        self.n_kq, self.r_k, self.n_vq, self.r_v, self.v_start = c.n_kq, c.r_k, c.n_vq, c.r_v, c.v_start
        self.last_launches = c.last_launches
        return out


class WindowCache:
    """WindowQuant cache of B x Hkv streams: reordered mixed-width windows + fp16 tail."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor, win_bits: torch.Tensor,
                 window_tokens: int, group: int, stream=None):
        """k, v: fp16 [B][Hkv][N][d] on the device; the first W*S tokens are the
        visual windows, the rest stays fp16.  win_bits: uint8 [W] on the device."""
        n, ss, rs = _streams(k)
        n2, ss2, rs2 = _streams(v)
        B, H, N, d = k.shape
        W = win_bits.numel()
        S = window_tokens
        self.B, self.H, self.d, self.G, self.S, self.W = B, H, d, group, S, W
        self.n_streams = n
        dev = k.device
        self.perm = torch.empty(W, dtype=torch.int32, device=dev)
        segs_dev = torch.zeros(4 * 32, dtype=torch.uint8, device=dev)
        n_segs = torch.zeros(1, dtype=torch.int32, device=dev)
        self.row_gather = torch.empty(W * S, dtype=torch.int32, device=dev)
        kvq_reorder_windows(win_bits, W, S, group, d, self.perm, segs_dev, n_segs,
                            self.row_gather, stream)
        ns = int(n_segs.cpu().item())          # synchronizes: the run table is needed on the host
        if ns < 0:
            raise ValueError("window bit widths must be 16, 8, 4 or 2")
        raw = segs_dev.cpu().numpy().tobytes()
        self.segs: List[Tuple[int, int, int, int, int]] = []
        for i in range(ns):
            s = Segment.from_buffer_copy(raw[32 * i: 32 * (i + 1)])
            self.segs.append(s.astuple())
        kc = km = vc = vm = 0
        for bits, t0, nt, coff, moff in self.segs:
            a, b_, c, e = arena_bytes(bits, nt, d, group)
            kc, km, vc, vm = max(kc, coff + a), max(km, moff + b_), max(vc, coff + c), max(vm, moff + e)
        u8 = dict(dtype=torch.uint8, device=dev)
        self.k_codes = torch.zeros(n, _round16(kc), **u8)
        self.k_meta = torch.zeros(n, max(16, _round16(km)), **u8)
        self.v_codes = torch.zeros(n, _round16(vc), **u8)
        self.v_meta = torch.zeros(n, max(16, _round16(vm)), **u8)
        for bits, t0, nt, coff, moff in self.segs:
            rows = self.row_gather[t0:t0 + nt]
            for which, src, s_, r_, codes, meta in (
                    (KVQ_KEYS, k, ss, rs, self.k_codes, self.k_meta),
                    (KVQ_VALUES, v, ss2, rs2, self.v_codes, self.v_meta)):
                kvq_quantize_append(which, bits, group, n, d, nt, src, s_, r_, rows,
                                    codes.data_ptr() + coff, codes.stride(0),
                                    meta.data_ptr() + moff, meta.stride(0), 0, stream)
        self.n_vis = W * S
        self.n_res = N - self.n_vis
        f16 = dict(dtype=torch.float16, device=dev)
        self.k_res = torch.zeros(n, max(self.n_res, 1), d, **f16)
        self.v_res = torch.zeros(n, max(self.n_res, 1), d, **f16)
        if self.n_res:
            kvq_residual_append(n, d, self.n_res, k[:, :, self.n_vis:], ss, rs, self.k_res,
                                self.k_res.stride(0), 0, stream)
            kvq_residual_append(n, d, self.n_res, v[:, :, self.n_vis:], ss2, rs2, self.v_res,
                                self.v_res.stride(0), 0, stream)
        self._ws = None

    def decode_args(self, q, out, sm_scale, split_tokens=0):
        B, Hq, d = q.shape
        a = make_decode_args(
            batch=B, n_q_heads=Hq, n_kv_heads=self.H, d_h=d, group=self.G, sm_scale=sm_scale, q=q,
            k_segs=self.segs, v_segs=self.segs,
            k_codes=self.k_codes, k_codes_stride=self.k_codes.stride(0),
            k_meta=self.k_meta, k_meta_stride=self.k_meta.stride(0),
            v_codes=self.v_codes, v_codes_stride=self.v_codes.stride(0),
            v_meta=self.v_meta, v_meta_stride=self.v_meta.stride(0),
            k_res=self.k_res, n_k_res=self.n_res, k_res_stride=self.k_res.stride(0),
            v_res=self.v_res, n_v_res=self.n_res, v_res_stride=self.v_res.stride(0),
            out=out, split_tokens=split_tokens)
        need = kvq_decode_attn_workspace(a)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        a.workspace = self._ws.data_ptr()
        a.workspace_bytes = self._ws.numel()
        return a

    def attend(self, q, sm_scale, out=None, split_tokens=0, stream=None):
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        kvq_decode_attn(self.decode_args(q, out, sm_scale, split_tokens), stream)
        return out


def kivi_step_lengths(context: int, residual: int) -> Tuple[int, int, int, int]:
    """(n_kq, r_k, n_vq, r_v) after a prefill of ``context`` tokens and one
    decode step (KIVI Algorithm 1): the prefill quantizes keys up to
    l - l % R and values up to l - R; the step appends one key (a full key
    residual of R is flushed) and one value (a window beyond R loses its
    oldest value to the quantized part)."""
    R = residual
    n_kq, r_k = context - context % R, context % R + 1
    if r_k == R:
        n_kq, r_k = n_kq + R, 0
    n_vq, r_v = max(context - R, 0), min(context, R) + 1
    if r_v > R:
        n_vq, r_v = n_vq + 1, R
    return n_kq, r_k, n_vq, r_v


class PagedKiviCache:
    """Paged, ragged KIVI cache of ``batch`` sequences x ``n_kv_heads`` heads.

    Sequence b's quantized keys and values live in pages of ``page_tokens``
    tokens (kvq_page_layout) taken from one pool in a shuffled order (so the
    block table is a real indirection); its fp16 key residual and value
    window are rows of per-stream buffers.  ``fill`` writes a sequence's state
    with the library's quantize and row-copy calls, one call per page.
    """

    def __init__(self, batch: int, n_kv_heads: int, d_h: int, bits: int, group: int, residual: int,
                 page_tokens: int, max_tokens: int, n_pages: Optional[int] = None, device="cuda",
                 seed: int = 0):
        self.B, self.H, self.d, self.bits, self.G, self.R = batch, n_kv_heads, d_h, bits, group, residual
        self.PT = page_tokens
        self.layout = kvq_page_layout(n_kv_heads, d_h, group, bits, page_tokens)
        self.max_pages = max(1, -(-max_tokens // page_tokens))
        n_pages = n_pages or batch * self.max_pages
        assert n_pages >= batch * self.max_pages
        self.page_bytes = self.layout["page_bytes"]
        self.pool = torch.zeros(n_pages, self.page_bytes, dtype=torch.uint8, device=device)
        order = torch.randperm(n_pages, generator=torch.Generator().manual_seed(seed))[:batch * self.max_pages]
        self.block_table_host = order.to(torch.int32).reshape(batch, self.max_pages)
        self.block_table = self.block_table_host.to(device)
        f16 = dict(dtype=torch.float16, device=device)
        self.n_streams = batch * n_kv_heads
        self.k_res = torch.zeros(self.n_streams, residual, d_h, **f16)
        self.v_res = torch.zeros(self.n_streams, residual + 1, d_h, **f16)
        self.lens = np.zeros((batch, 4), dtype=np.int32)      # n_kq, n_vq, n_k_res, n_v_res
        self.lens_dev = torch.zeros(batch, 4, dtype=torch.int32, device=device)
        self._ws = None

    def _page_ptr(self, b: int, j: int, part: str) -> int:
        off = {"kcodes": 0, "kmeta": self.layout["kmeta_off"], "vcodes": self.layout["vcodes_off"],
               "vmeta": self.layout["vmeta_off"]}[part]
        return self.pool.data_ptr() + int(self.block_table_host[b, j]) * self.page_bytes + off

    def fill(self, b: int, k: torch.Tensor, v: torch.Tensor, n_kq: int, n_vq: int, stream=None):
        """Sequence b holds tokens k, v [Hkv][N][d] (fp16, on the device): keys
        0..n_kq-1 and values 0..n_vq-1 quantized into its pages (one
        kvq_quantize_append per page and half; a page is a key run and a
        value run of its kv heads), the rest copied to the residual rows."""
        H, d, PT, hb = self.H, self.d, self.PT, self.layout["head_bytes"]
        assert k.shape == v.shape and k.shape[0] == H and k.shape[2] == d and k.dtype == torch.float16
        N = k.shape[1]
        assert n_kq % self.G == 0 and 0 <= n_vq <= n_kq <= N and N - n_kq <= self.R and N - n_vq <= self.R + 1
        assert -(-n_kq // PT) <= self.max_pages
        for which, src, n_q, codes, meta in ((KVQ_KEYS, k, n_kq, "kcodes", "kmeta"),
                                             (KVQ_VALUES, v, n_vq, "vcodes", "vmeta")):
            for j in range(-(-n_q // PT)):
                t0, t1 = j * PT, min(n_q, (j + 1) * PT)
                kvq_quantize_append(which, self.bits, self.G, H, d, t1 - t0, src[:, t0:], src.stride(0),
                                    src.stride(1), None, self._page_ptr(b, j, codes), hb,
                                    self._page_ptr(b, j, meta), hb, 0, stream)
        s0 = b * H
        if N > n_kq:
            kvq_residual_append(H, d, N - n_kq, k[:, n_kq:], k.stride(0), k.stride(1), self.k_res[s0],
                                self.k_res.stride(0), 0, stream)
        if N > n_vq:
            kvq_residual_append(H, d, N - n_vq, v[:, n_vq:], v.stride(0), v.stride(1), self.v_res[s0],
                                self.v_res.stride(0), 0, stream)
        self.lens[b] = (n_kq, n_vq, N - n_kq, N - n_vq)
        self.lens_dev[b].copy_(torch.from_numpy(self.lens[b].copy()))

    def fill_step(self, b: int, k: torch.Tensor, v: torch.Tensor, stream=None):
        """The state of sequence b after a prefill of N - 1 tokens and one
        decode step (kivi_step_lengths) for k, v [Hkv][N][d]."""
        n_kq, _, n_vq, _ = kivi_step_lengths(k.shape[1] - 1, self.R)
        self.fill(b, k, v, n_kq, n_vq, stream)

    def args(self, q: torch.Tensor, sm_scale: float, out: torch.Tensor) -> PagedArgs:
        a = PagedArgs()
        a.batch, a.n_q_heads, a.n_kv_heads = self.B, q.shape[1], self.H
        a.d_h, a.group, a.bits, a.sm_scale, a.page_tokens = self.d, self.G, self.bits, float(sm_scale), self.PT
        a.q, a.pages, a.page_bytes = q.data_ptr(), self.pool.data_ptr(), self.page_bytes
        a.block_table, a.max_pages = self.block_table.data_ptr(), self.max_pages
        a.lengths = self.lens.ctypes.data
        a.lengths_dev = self.lens_dev.data_ptr()
        a.k_res, a.k_res_stride = self.k_res.data_ptr(), self.k_res.stride(0)
        a.v_res, a.v_res_stride = self.v_res.data_ptr(), self.v_res.stride(0)
        a.out = out.data_ptr()
        return a

    def attend(self, q: torch.Tensor, sm_scale: float, out: Optional[torch.Tensor] = None, stream=None):
        """kvq_decode_attn_paged of q [B][Hq][d] (fp16) over every sequence."""
        assert q.dtype == torch.float16 and q.is_contiguous()
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        a = self.args(q, sm_scale, out)
        need = kvq_decode_attn_paged_workspace(a)
        if need and (self._ws is None or self._ws.numel() < need):
            self._ws = torch.empty(need, dtype=torch.uint8, device=q.device)
        if need:
            a.workspace, a.workspace_bytes = self._ws.data_ptr(), self._ws.numel()
        kvq_decode_attn_paged(a, stream)
        return out
