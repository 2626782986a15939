"""PQCache decode-time PQ search (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
path imports this module.

PQCache note, "Background" (product quantization) and "Method details",
Steps 2 and 4:

* a key vector of d_h channels is cut into m sub-vectors of d_m = d_h / m
  channels; each sub-space j has 2^b centroids of d_m channels (shape
  (m, 2^b, d_m) per head) and every token carries m codes of b bits (shape
  (s, m)), code j naming its sub-vector's centroid;
* decode-time search: multiply the query with the centroids (one table of
  q_j . centroid[j][c] per sub-space j and centroid c), then aggregate the
  table entries named by each token's codes: the approximate score of token
  t is the dot product of the query with the key rebuilt from its centroids;
* the Top-k tokens by approximate score are the ones whose key/value pairs
  are then fetched for attention.

Readings where the page is silent:

* scores are the raw dot products q . k~ (no 1/sqrt(d_h): the ranking is the
  same), in float64 here;
* GQA: query head hq uses the PQ of kv head hq // (Hq / Hkv) (the pages'
  grouped heads share one key cache);
* Top-k: the k tokens with the largest scores, ties to the lower token index,
  returned in ascending token order;
* centroids and codes are inputs (PQ construction is K-means on the host,
  outside this path).
"""
from __future__ import annotations

import numpy as np

__all__ = ["score_tables", "pq_scores", "topk_tokens", "pq_search"]


def score_tables(q: np.ndarray, centroids: np.ndarray) -> np.ndarray:
    """Per sub-space j and centroid c: q_j . centroid[j][c] (float64 [m][2^b]).

    q: [d_h]; centroids: [m][2^b][d_m] with m * d_m = d_h."""
    m, nc, dm = centroids.shape
    qs = np.asarray(q, np.float64).reshape(m, dm)
    return np.einsum("jd,jcd->jc", qs, np.asarray(centroids, np.float64))


def pq_scores(q: np.ndarray, centroids: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """Approximate score of every token: sum over j of table[j][codes[t][j]]
    (float64 [s]); codes: [s][m] integers."""
    t = score_tables(q, centroids)
    codes = np.asarray(codes, np.int64)
    s, m = codes.shape
    out = np.zeros(s, np.float64)
    for j in range(m):
        out += t[j][codes[:, j]]
    return out


def topk_tokens(scores: np.ndarray, k: int) -> np.ndarray:
    """The k tokens with the largest scores (ties to the lower index), in
    ascending token order (int64 [k])."""
    scores = np.asarray(scores)
    k = min(k, scores.shape[0])
    order = sorted(range(scores.shape[0]), key=lambda t: (-scores[t], t))
    return np.array(sorted(order[:k]), dtype=np.int64)


def pq_search(q: np.ndarray, centroids: np.ndarray, codes: np.ndarray, k: int):
    """(scores [s], top-k token indices [k]) of one query head."""
    sc = pq_scores(q, centroids, codes)
    return sc, topk_tokens(sc, k)
