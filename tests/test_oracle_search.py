"""Pins of the oracle's WindowQuant window-level search (Sec. 3.2).

* hand-derived score, thresholds and votes (tests/golden/search_examples.json);
* Eq. 10-11 closed-form properties the page states (both thresholds run from
  0 to 1, T_low <= T_high on [0, 1]), the identity T_high(s) = 1 - T_low(1 - s)
  and the alpha -> 0 limit (both -> s);
* Eq. 8 against explicit loops over every (text, visual) token pair, against
  plain cosines when N = S = 1, and its invariances (positive scaling of any
  token, negation of the prompt, trailing tokens that are no window);
* the decision rule at and around the thresholds, the first-window rule.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import search
from tests.test_gpu_search import MARGIN, admissible

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "search_examples.json")))


def test_golden_score_thresholds_votes():
    e = GOLD["score_example"]
    s = search.window_scores(np.array(e["text"]), np.array(e["visual"]), e["S"])
    assert s.shape == (1,) and abs(s[0] - e["score"]) < 1e-15
    t = GOLD["threshold_example"]
    lo, hi = search.thresholds(t["s"], t["alpha"])
    assert abs(lo - t["t_low"]) < 1e-15 and abs(hi - t["t_high"]) < 1e-15
    for v in GOLD["vote_examples"]:
        assert search.batch_vote(v["choices"]) == v["bits"], v["why"]


@pytest.mark.parametrize("alpha", [0.5, 2.0, 5.0, -3.0])
def test_thresholds_properties(alpha):
    lo0, hi0 = search.thresholds(0.0, alpha)
    lo1, hi1 = search.thresholds(1.0, alpha)
    assert lo0 == 0.0 and hi0 == 0.0
    assert abs(lo1 - 1.0) < 1e-15 and abs(hi1 - 1.0) < 1e-15
    for s in np.linspace(0, 1, 101):
        lo, hi = search.thresholds(s, alpha)
        lo_m, _ = search.thresholds(1 - s, alpha)
        assert abs(hi - (1 - lo_m)) < 1e-12              # T_high(s) = 1 - T_low(1 - s)
        if alpha > 0:
            assert lo <= hi + 1e-15                       # the page's ordering on [0, 1]
    lo, hi = search.thresholds(0.3, 1e-7)
    assert abs(lo - 0.3) < 1e-6 and abs(hi - 0.3) < 1e-6  # alpha -> 0: both -> s


def test_scores_against_explicit_pair_loops():
    rng = np.random.default_rng(3)
    for _ in range(10):
        N, S, W, D = (int(x) for x in rng.integers(1, 6, size=4))
        text = rng.standard_normal((N, D))
        vis = rng.standard_normal((W * S + int(rng.integers(0, S)), D))
        got = search.window_scores(text, vis, S)
        assert got.shape == (W,)
        for i in range(W):
            tot = 0.0
            for j in range(N):
                for k in range(S):
                    a, b = text[j], vis[i * S + k]
                    tot += float(np.dot(a, b)) / (math.sqrt(float(np.dot(a, a))) * math.sqrt(float(np.dot(b, b))))
            assert abs(got[i] - tot / (N * S)) < 1e-12


def test_scores_plain_cosine_and_invariances():
    rng = np.random.default_rng(4)
    a, b = rng.standard_normal(7), rng.standard_normal(7)
    s = search.window_scores(a[None], b[None], 1)[0]
    assert abs(s - a @ b / np.linalg.norm(a) / np.linalg.norm(b)) < 1e-14
    text = rng.standard_normal((5, 16))
    vis = rng.standard_normal((4 * 8, 16))
    base = search.window_scores(text, vis, 8)
    scaled = vis * rng.uniform(0.01, 100, size=(vis.shape[0], 1))
    assert np.allclose(search.window_scores(text * 3.0, scaled, 8), base, atol=1e-14, rtol=0)
    assert np.allclose(search.window_scores(-text, vis, 8), -base, atol=1e-14, rtol=0)
    extra = np.concatenate([vis, rng.standard_normal((7, 16))])
    assert np.array_equal(search.window_scores(text, extra, 8), base)
    # identical directions score 1, a zero token contributes a zero cosine
    u = rng.standard_normal(16)
    assert abs(search.window_scores(u[None], np.stack([u, 2 * u]), 2)[0] - 1.0) < 1e-14
    assert abs(search.window_scores(u[None], np.stack([u, 0 * u]), 2)[0] - 0.5) < 1e-14


def test_decision_rule_and_first_window():
    assert search.choose_bits(0.8, 0.3, 0.7) == 16
    assert search.choose_bits(0.7, 0.3, 0.7) == 4      # equal: not above T_high
    assert search.choose_bits(0.3, 0.3, 0.7) == 4      # equal: not below T_low
    assert search.choose_bits(0.29, 0.3, 0.7) == 2
    rng = np.random.default_rng(5)
    text = rng.standard_normal((2, 3, 8))
    vis = rng.standard_normal((2, 5 * 4, 8))
    sc, bits = search.search(text, vis, 4, 10.0, 20.0)           # every score below T_low
    assert bits.tolist() == [16, 2, 2, 2, 2] and sc.shape == (2, 5)
    _, bits = search.search(text, vis, 4, 10.0, 20.0, first_window_fp16=False)
    assert bits.tolist() == [2] * 5
    _, bits = search.search(text, vis, 4, -10.0, -5.0)            # every score above T_high
    assert bits.tolist() == [16] * 5


def test_admissible_set_rule():
    """The GPU window-search test's admissible sets (CPU arithmetic): one width far
    from the thresholds, the two neighbours of a near threshold only, and the
    vote over the rows' combinations."""
    lo, hi = 0.3, 0.6
    assert admissible([0.1], lo, hi, False) == {2}
    assert admissible([0.45], lo, hi, False) == {4}
    assert admissible([0.9], lo, hi, False) == {16}
    assert admissible([lo - MARGIN / 2], lo, hi, False) == {2, 4}
    assert admissible([hi + MARGIN / 2], lo, hi, False) == {4, 16}
    assert admissible([0.1, 0.9, lo + MARGIN / 2], lo, hi, False) == {2, 16}   # 2/16/{2,4}: 2 wins 2-1, or a 3-way tie -> 16
    assert admissible([0.1, 0.1, hi + MARGIN / 2], lo, hi, False) == {2}
    assert admissible([0.1], lo, hi, True) == {16}

