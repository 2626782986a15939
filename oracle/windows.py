"""WindowQuant window reorder and per-window quantization (oracle).

WindowQuant (ACM TACO), Sec. 3.1 and 3.3.1: after the first output token of
prefill, the KV windows are rearranged so that windows with the same bit
width sit next to each other in memory, and each window is then quantized at
its assigned width.  Sec. 3.3.2 (Eq. 12-13) shows the decode output does not
depend on the window order, since decode applies no mask.  Text tokens (and
generated tokens) stay fp16 (Sec. 3.1).

Readings taken:

* order of the runs: descending bit width, 16 > 8 > 4 > 2; inside a run,
  ascending original window index (a stable sort), perm[new] = old;
* quantization inside a window uses KIVI's axes and the group size G of the
  call (keys per channel over G tokens, values per token over G channels),
  G dividing the window size; WindowQuant's own group-per-window reading is
  the special case G = S for keys;
* each run's place in a stream's arena follows the header's rule: runs are
  laid out in order, each starting at the previous run's end rounded up to
  256 bytes, for codes and for (scale, zero) pairs separately.
"""
from __future__ import annotations

from typing import List, NamedTuple

import numpy as np

from .quant import (quantize_keys, quantize_values, dequantize_keys,
                    dequantize_values)
from .attention import blocks_attention

__all__ = ["Segment", "reorder", "segment_table", "row_gather",
           "WindowStream", "attend_in_place"]

BIT_ORDER = (16, 8, 4, 2)
ALIGN = 256


class Segment(NamedTuple):
    bits: int
    tok_begin: int
    n_tok: int
    code_off: int
    meta_off: int


def reorder(win_bits) -> List[int]:
    """Stable sort of windows by descending bit width: perm[new] = old."""
    return sorted(range(len(win_bits)), key=lambda i: (-int(win_bits[i]), i))


def _align(x: int) -> int:
    return (x + ALIGN - 1) // ALIGN * ALIGN


def code_bytes(bits: int, n_tok: int, d: int) -> int:
    return n_tok * d * (2 if bits == 16 else bits) // (1 if bits == 16 else 8)


def meta_bytes(bits: int, n_tok: int, d: int, group: int) -> int:
    return 0 if bits == 16 else n_tok * (d // group) * 4


def segment_table(win_bits, window_tokens: int, d: int, group: int) -> List[Segment]:
    """One run per bit width present, in the reorder's order."""
    segs, tok, coff, moff = [], 0, 0, 0
    for b in BIT_ORDER:
        n_win = int(sum(1 for x in win_bits if int(x) == b))
        if n_win == 0:
            continue
        n = n_win * window_tokens
        segs.append(Segment(b, tok, n, coff, moff))
        tok += n
        coff = _align(coff + code_bytes(b, n, d))
        moff = _align(moff + meta_bytes(b, n, d, group))
    return segs


def row_gather(perm, window_tokens: int) -> np.ndarray:
    """Source token of every reordered token: perm[w]*S + i at w*S + i."""
    s = window_tokens
    return np.array([perm[w] * s + i for w in range(len(perm)) for i in range(s)],
                    dtype=np.int32)


class WindowStream:
    """One (batch, kv-head) stream: reordered quantized windows + fp16 tail."""

    def __init__(self, xk, xv, win_bits, window_tokens: int, group: int):
        """xk, xv fp16 [N][d]; the first W*S tokens are the visual windows,
        the rest (text tokens and the decode token) stay fp16."""
        d = xk.shape[1]
        s = window_tokens
        n_vis = len(win_bits) * s
        self.group = group
        self.perm = reorder(win_bits)
        self.segs = segment_table(win_bits, s, d, group)
        gather = row_gather(self.perm, s)
        self.runs = []   # (bits, key part, value part) per segment
        for seg in self.segs:
            rows = gather[seg.tok_begin: seg.tok_begin + seg.n_tok]
            k, v = xk[rows], xv[rows]
            if seg.bits == 16:
                self.runs.append((16, k.copy(), v.copy()))
            else:
                self.runs.append((seg.bits, quantize_keys(k, seg.bits, group),
                                  quantize_values(v, seg.bits, group)))
        self.k_res = xk[n_vis:].copy()
        self.v_res = xv[n_vis:].copy()

    def _blocks(self):
        kb, vb = [], []
        for bits, kp, vp in self.runs:
            if bits == 16:
                kb.append(kp.astype(np.float64))
                vb.append(vp.astype(np.float64))
            else:
                kb.append(dequantize_keys(*kp, self.group))
                vb.append(dequantize_values(*vp, self.group))
        return kb + [self.k_res], vb + [self.v_res]

    def attend(self, q, sm_scale: float) -> np.ndarray:
        kb, vb = self._blocks()
        return blocks_attention(q, kb, vb, sm_scale)


def attend_in_place(xk, xv, win_bits, window_tokens: int, group: int, q,
                    sm_scale: float) -> np.ndarray:
    """Mixed-precision attention *without* the reorder: every window is
    quantized where it stands and the blocks stay in token order."""
    s = window_tokens
    n_vis = len(win_bits) * s
    kb, vb = [], []
    for w, b in enumerate(win_bits):
        k, v = xk[w * s:(w + 1) * s], xv[w * s:(w + 1) * s]
        if int(b) == 16:
            kb.append(k.astype(np.float64))
            vb.append(v.astype(np.float64))
        else:
            kb.append(dequantize_keys(*quantize_keys(k, int(b), group), group))
            vb.append(dequantize_values(*quantize_values(v, int(b), group), group))
    return blocks_attention(q, kb + [xk[n_vis:]], vb + [xv[n_vis:]], sm_scale)
