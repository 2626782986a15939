"""KIVI cache state machine (oracle), one (batch, kv-head) stream at a time.

Follows the KIVI note's Algorithm 1 ("Appendix details") and "Method details":

* Prefill: values X_V[:l-R] are quantized per token, the last R stay fp16;
  keys go through KeyQuant: r = l % R, X_K[:l-r] quantized per channel in
  groups of G tokens, X_K[l-r:] stay fp16.
* Decoding: the new token's key and value are appended to the fp16
  residuals; when the key residual reaches R tokens it is quantized as a
  whole, appended to the grouped keys and emptied; when the value residual
  holds more than R tokens its oldest tokens are quantized per token and
  appended, and the residual keeps the last R.
* Attention: one softmax over [grouped-key logits, residual-key logits]; the
  probabilities multiply [dequantized grouped values, residual values].

Readings taken where the pages are silent:

* prefill with l < R keeps every value token in the residual (the slice
  X_V[:l-R] is read as empty, not as Python's negative index);
* R must be a multiple of G (the pages require it) so every flushed key
  chunk is whole groups.
"""
from __future__ import annotations

import numpy as np

from .quant import (quantize_keys, quantize_values, dequantize_keys,
                    dequantize_values)
from .attention import blocks_attention

__all__ = ["KiviStream", "kivi_lengths"]


class KiviStream:
    """Quantized keys/values, fp16 residuals and their (s, z) for one stream."""

    def __init__(self, d: int, bits: int, group: int, residual: int):
        assert residual % group == 0 and d % group == 0
        self.d, self.bits, self.G, self.R = d, bits, group, residual
        u8, f16 = np.uint8, np.float16
        self.kq = np.zeros((0, d), u8)
        self.ks = np.zeros((0, d), f16)
        self.kz = np.zeros((0, d), f16)
        self.k_res = np.zeros((0, d), f16)
        self.vq = np.zeros((0, d), u8)
        self.vs = np.zeros((0, d // group), f16)
        self.vz = np.zeros((0, d // group), f16)
        self.v_res = np.zeros((0, d), f16)

    # -- KeyQuant / GroupQuant -------------------------------------------------
    def _key_quant(self, xk: np.ndarray):
        """KeyQuant: quantize the first l - l%R tokens, return the rest."""
        l = xk.shape[0]
        r = l % self.R
        codes, s, z = quantize_keys(xk[: l - r], self.bits, self.G)
        self.kq = np.concatenate([self.kq, codes])
        self.ks = np.concatenate([self.ks, s])
        self.kz = np.concatenate([self.kz, z])
        return xk[l - r:]

    def _value_quant(self, xv: np.ndarray):
        codes, s, z = quantize_values(xv, self.bits, self.G)
        self.vq = np.concatenate([self.vq, codes])
        self.vs = np.concatenate([self.vs, s])
        self.vz = np.concatenate([self.vz, z])

    # -- Algorithm 1 ------------------------------------------------------------
    def prefill(self, xk: np.ndarray, xv: np.ndarray) -> None:
        l = xk.shape[0]
        n_vq = max(l - self.R, 0)
        self._value_quant(xv[:n_vq])
        self.v_res = xv[n_vq:].copy()
        self.k_res = self._key_quant(xk).copy()

    def decode_append(self, tk: np.ndarray, tv: np.ndarray) -> None:
        self.k_res = np.concatenate([self.k_res, tk.reshape(1, -1)])
        self.v_res = np.concatenate([self.v_res, tv.reshape(1, -1)])
        if self.k_res.shape[0] == self.R:
            rest = self._key_quant(self.k_res)
            assert rest.shape[0] == 0
            self.k_res = rest
        if self.v_res.shape[0] > self.R:
            self._value_quant(self.v_res[:-self.R])
            self.v_res = self.v_res[-self.R:].copy()

    @property
    def lengths(self):
        """(n_Kq, r_K, n_Vq, r_V): tokens in each of the four cache parts."""
        return (self.kq.shape[0], self.k_res.shape[0],
                self.vq.shape[0], self.v_res.shape[0])

    def attend(self, q: np.ndarray, sm_scale: float) -> np.ndarray:
        """Decode attention of the query heads q [g][d] over this stream."""
        kq = dequantize_keys(self.kq, self.ks, self.kz, self.G)
        vq = dequantize_values(self.vq, self.vs, self.vz, self.G)
        return blocks_attention(q, [kq, self.k_res], [vq, self.v_res], sm_scale)


def kivi_lengths(l_prefill: int, n_decode: int, residual: int):
    """Cache part sizes after prefill of l tokens and n decode steps.

    A direct count, not a simulation: keys are quantized in whole chunks of R
    and the key residual holds the remainder; values keep the last R tokens in
    fp16.
    """
    total = l_prefill + n_decode
    n_kq = residual * (total // residual)
    n_vq = max(total - residual, 0)
    return n_kq, total - n_kq, n_vq, total - n_vq
