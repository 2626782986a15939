"""Decode attention over a vector-quantized (codebook) KV cache (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
path imports this module.

VQ-LLM note, "Background" on vector quantization and the CQ-2 / CQ-4 KV-cache
configurations it evaluates (the CQ reference: every four channels switch to
their own codebook):

* a vector is cut into sub-vectors; each sub-vector is replaced by the index
  of a codebook entry; the residual between the sub-vector and that entry
  may be quantized again with a further codebook (residual rounds);
* dequantization looks the entries up, adds the residual rounds element by
  element and concatenates the sub-spaces;
* decode attention then runs over the dequantized keys and values like any
  other attention: one softmax over the scaled logits of the query with
  every key, and the probability-weighted sum of the values.

Readings where the page is silent or loose:

* sub-vectors are groups of 4 consecutive channels (d_h / 4 groups), each
  with its own codebook of 256 entries (8-bit codes; the page's CQ-2
  microbenchmark has 256-entry codebooks), separately for keys and values,
  per kv head, shared by every sequence of the batch;
* CQ-2 is one round (8 bits per 4 channels: 2 bits per channel, the 1/8
  compression the page quotes); CQ-4 is two rounds, the second coding the
  residual of the first (4 bits per channel);
* every cached token is coded (the pages give VQ no full-precision window);
* GQA: query head hq attends kv head hq // (Hq / Hkv), as for KIVI;
* the score scale is an argument (the workloads use 1/sqrt(d_h)).

Everything here is float64 (codebooks are fp16 inputs, widened exactly).
"""
from __future__ import annotations

import numpy as np

from . import attention

__all__ = ["dequantize", "vq_attention"]


def dequantize(codes: np.ndarray, books: np.ndarray) -> np.ndarray:
    """codes uint8 [n][R][G]; books [R][G][E][c] -> float64 [n][G * c].

    Row t, channels g*c .. g*c+c-1: the sum over rounds r of the entry
    books[r][g][codes[t][r][g]].
    """
    codes = np.asarray(codes)
    books = np.asarray(books, dtype=np.float64)
    n, R, G = codes.shape
    assert books.shape[:2] == (R, G), (books.shape, codes.shape)
    c = books.shape[3]
    out = np.zeros((n, G, c), dtype=np.float64)
    for r in range(R):
        for g in range(G):
            out[:, g, :] += books[r, g][codes[:, r, g].astype(np.int64)]
    return out.reshape(n, G * c)


def vq_attention(q: np.ndarray, k_codes: np.ndarray, v_codes: np.ndarray, k_books: np.ndarray,
                 v_books: np.ndarray, sm_scale: float) -> np.ndarray:
    """q [g][d] (the query heads of one kv head); codes [n][R][G] of that kv
    head's keys and values; books [R][G][E][c].  Returns float64 [g][d]."""
    k = dequantize(k_codes, k_books)
    v = dequantize(v_codes, v_books)
    return attention.blocks_attention(q, [k], [v], sm_scale)
