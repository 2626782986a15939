"""Single-query softmax attention over blocks of keys and values (oracle).

KIVI note, "Method details": the logits of the quantized part and of the
full-precision residual are computed separately and concatenated,
A = Concat([t_Q Q(X_Kg)^T, t_Q X_Kr^T]); one softmax runs over the whole
concatenation and the output is the probability-weighted sum of the
(dequantized) value rows, t_O = A_g Q(X_Vg) + A_r X_Vr (Algorithm 1,
Decoding).

WindowQuant Sec. 3.3.1 describes the same computation over several bit-width
blocks: Q times each block's K^T, concatenate along the token axis, softmax
(no mask in decode), split the probabilities again and sum the per-block
products with V.

Reading taken for the split (Algorithm 1 slices the probability vector by
the residual length R): the probability vector is split at the *value*
blocks' boundaries, which need not coincide with the key blocks'
boundaries, because keys and values flush at different times.

Score scale: the KIVI note writes t_Q X_K^T without a scale; the VQ-LLM and
WindowQuant pages (Eq. 2) divide by sqrt(d_k).  The scale is an argument,
``sm_scale``; the workloads use 1/sqrt(d_h).

Everything here is float64.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

__all__ = ["blocks_attention"]


def blocks_attention(q: np.ndarray, k_blocks: Sequence[np.ndarray],
                     v_blocks: Sequence[np.ndarray], sm_scale: float) -> np.ndarray:
    """q [g][d] (query heads sharing this kv stream); blocks [n_i][d].

    Returns float64 [g][d].
    """
    q64 = np.asarray(q, dtype=np.float64)
    logits = [q64 @ np.asarray(kb, dtype=np.float64).T for kb in k_blocks]
    a = np.concatenate(logits, axis=1) * float(sm_scale)       # [g][N]
    n_v = sum(vb.shape[0] for vb in v_blocks)
    assert a.shape[1] == n_v, "keys and values must cover the same tokens"
    a = a - a.max(axis=1, keepdims=True)
    p = np.exp(a)
    p /= p.sum(axis=1, keepdims=True)
    out = np.zeros((q64.shape[0], q64.shape[1]), dtype=np.float64)
    start = 0
    for vb in v_blocks:
        n = vb.shape[0]
        out += p[:, start:start + n] @ np.asarray(vb, dtype=np.float64)
        start += n
    return out
