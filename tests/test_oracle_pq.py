"""Pins of the PQ-search oracle (oracle/pq.py) against what the PQCache note
fixes: the hand-derived example in tests/golden/pq_examples.json, the
reconstruction identity (an approximate score is the query's dot product
with the key rebuilt from the centroids), exactness when every key is its
own centroid, and a brute-force Top-k with the tie rule."""
import json
import os

import numpy as np

from oracle import pq

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pq_examples.json")


def test_hand_derived_example():
    g = json.load(open(GOLDEN))
    q = np.array(g["q"])
    c = np.array(g["centroids"])
    codes = np.array(g["codes"])
    assert np.array_equal(pq.score_tables(q, c), np.array(g["tables"]))
    assert np.array_equal(pq.pq_scores(q, c, codes), np.array(g["scores"]))
    assert pq.topk_tokens(pq.pq_scores(q, c, codes), 2).tolist() == g["top2"]
    assert pq.pq_search(q, c, codes, 3)[1].tolist() == g["top3"]


def test_reconstruction_identity():
    # the table lookup equals q . k~ with k~ = concat_j centroid[j][code_tj]
    rng = np.random.default_rng(0)
    for m, bits, dm in ((1, 4, 64), (2, 8, 64), (4, 6, 32), (8, 3, 16)):
        c = rng.standard_normal((m, 1 << bits, dm))
        codes = rng.integers(0, 1 << bits, size=(300, m))
        q = rng.standard_normal(m * dm)
        rebuilt = np.concatenate([c[j][codes[:, j]] for j in range(m)], axis=1)   # [s][d_h]
        assert np.allclose(pq.pq_scores(q, c, codes), rebuilt @ q, rtol=0, atol=1e-12)


def test_exact_when_keys_are_their_own_centroids():
    # 2^b >= s and centroid j of sub-space i = token j's sub-vector: PQ loses
    # nothing, so the scores are the exact q . k and Top-k is the exact one
    rng = np.random.default_rng(1)
    s, m, dm = 64, 4, 32
    keys = rng.standard_normal((s, m * dm))
    c = keys.reshape(s, m, dm).transpose(1, 0, 2).copy()     # [m][2^b = s][dm]
    codes = np.repeat(np.arange(s)[:, None], m, axis=1)
    q = rng.standard_normal(m * dm)
    sc = pq.pq_scores(q, c, codes)
    assert np.allclose(sc, keys @ q, atol=1e-12)
    assert pq.topk_tokens(sc, 10).tolist() == sorted(np.argsort(-(keys @ q), kind="stable")[:10].tolist())


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(2)
    for s, k in ((1, 1), (7, 3), (100, 10), (100, 100), (257, 31)):
        sc = rng.integers(-5, 6, size=s).astype(np.float64)    # many ties
        got = pq.topk_tokens(sc, k)
        order = np.lexsort((np.arange(s), -sc))                 # score desc, then index asc
        assert got.tolist() == sorted(order[:k].tolist())
        chosen = set(got.tolist())
        worst_in = min((sc[t], -t) for t in chosen)
        assert all((sc[u], -u) < worst_in for u in range(s) if u not in chosen)
    assert pq.topk_tokens(np.array([3.0, 1.0]), 5).tolist() == [0, 1]   # k > s: every token
