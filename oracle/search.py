"""WindowQuant window-level quantization search (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
path imports this module.

WindowQuant (ACM TACO), Sec. 3.2 "window-level quantization search":

* Eq. 8: the score of visual window i against the text prompt is the mean,
  over every pair (text token j, visual token k of the window), of the cosine
  similarity of the two token vectors;
* Sec. 3.2.1: a score above T_high keeps the window's KV cache in fp16, a score
  below T_low quantizes it to int2, anything in between to int4;
* Sec. 3.2.2: the first window stays fp16 whatever its score;
* Eq. 10-11: the thresholds of a layer follow from that layer's hidden-state
  similarity s (Eq. 9) and a hyper-parameter alpha:
  T_low = (e^{alpha s} - 1) / (e^{alpha} - 1),
  T_high = (e^{-alpha s} - 1) / (e^{-alpha} - 1);
* Sec. 3.2.3 (batched requests): every request of a batch gets the same
  configuration; per window, the width chosen most often over the batch.

Readings where the page is silent:

* windows are the floor(M/S) full windows of S visual tokens; trailing visual
  tokens are not a window and stay fp16 (Sec. 3.1);
* a token vector of zero length has no direction: its cosines count as 0;
* comparisons are strict as worded ("above T_high", "below T_low"): a score
  equal to a threshold gets int4;
* a vote tie goes to the wider width (the page names no rule; the wider one
  loses no information);
* scores in float64 (the page fixes no precision).
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np

__all__ = ["thresholds", "unit_rows", "window_scores", "choose_bits", "batch_vote", "search"]

WIDTHS = (16, 4, 2)


def thresholds(layer_similarity: float, alpha: float) -> Tuple[float, float]:
    """(T_low, T_high) of a layer, Eq. 10 and Eq. 11 (alpha != 0)."""
    s, a = float(layer_similarity), float(alpha)
    t_low = (math.exp(a * s) - 1.0) / (math.exp(a) - 1.0)
    t_high = (math.exp(-a * s) - 1.0) / (math.exp(-a) - 1.0)
    return t_low, t_high


def unit_rows(x: np.ndarray) -> np.ndarray:
    """Rows of x scaled to unit L2 length in float64; zero rows stay zero."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.divide(x, n, out=np.zeros_like(x), where=n > 0)


def window_scores(text: np.ndarray, visual: np.ndarray, window_tokens: int) -> np.ndarray:
    """Eq. 8 for one request: text [N][D], visual [M][D] -> scores [M // S].

    Each window's score is the mean of its full N x S matrix of pairwise
    cosines (text unit rows times window unit rows)."""
    S = int(window_tokens)
    t = unit_rows(text)
    v = unit_rows(visual)
    n_win = v.shape[0] // S
    out = np.empty(n_win, dtype=np.float64)
    for i in range(n_win):
        cos = t @ v[i * S:(i + 1) * S].T          # [N][S] pairwise cosines
        out[i] = cos.mean() if cos.size else 0.0
    return out


def choose_bits(score: float, t_low: float, t_high: float) -> int:
    """Sec. 3.2.1: fp16 above T_high, int2 below T_low, int4 otherwise."""
    if score > t_high:
        return 16
    if score < t_low:
        return 2
    return 4


def batch_vote(choices) -> int:
    """Sec. 3.2.3: the width chosen most often; ties to the wider width."""
    counts = {b: 0 for b in WIDTHS}
    for c in choices:
        counts[int(c)] += 1
    return max(WIDTHS, key=lambda b: (counts[b], b))


def search(text: np.ndarray, visual: np.ndarray, window_tokens: int, t_low: float, t_high: float,
           first_window_fp16: bool = True):
    """Whole search for a batch: text [B][N][D], visual [B][M][D] ->
    (scores [B][W] float64, win_bits [W] uint8)."""
    text = np.asarray(text)
    visual = np.asarray(visual)
    B = text.shape[0]
    scores = np.stack([window_scores(text[b], visual[b], window_tokens) for b in range(B)])
    W = scores.shape[1]
    bits = np.empty(W, dtype=np.uint8)
    for i in range(W):
        bits[i] = batch_vote([choose_bits(scores[b, i], t_low, t_high) for b in range(B)])
    if first_window_fp16 and W > 0:
        bits[0] = 16
    return scores, bits
