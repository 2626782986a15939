"""GPU parity of the WindowQuant window-level search (kvq_window_search)
against the oracle (WindowQuant Sec. 3.2).

* scores within 2e-5 of the float64 oracle (the kernel sums fp32 unit
  vectors; the oracle averages the full matrix of pairwise cosines);
* window widths in the set the oracle's rule admits: per batch row, every
  width the decision rule gives for a score within 1e-4 of the oracle's
  (one width unless a threshold is that close: then the two widths on
  either side of it, and only those), and per window the vote over every
  combination of the rows' admissible widths; so a window far from both
  thresholds must get exactly the oracle's width, and one near T_low can
  never get 16 (nor one near T_high 2);
* scores placed just below T_low and just above T_high on purpose;
* shapes with partial 64-token chunks, trailing tokens that are no window,
  one text token, zero-length rows, dims 8 .. 4096 and batches of 1 .. 5;
* the first-window rule both ways, repeated calls bit-identical, and the
  full-size case (128 windows of 256 tokens, dim 3584) at the batch size the
  pages' VLM workloads use.
"""
import itertools

import numpy as np
import pytest

import workloads
from oracle import search
from tests.helpers import ensure_built

pytestmark = pytest.mark.gpu

SCORE_TOL = 2e-5
MARGIN = 1e-4


@pytest.fixture(scope="module")
def kvq():
    ensure_built()
    import decode_attention_kivi_amd as m
    return m


def run_search(kvq, text, visual, S, t_low, t_high, first=True, text_pad=0, vis_pad=0):
    import torch
    B, N, D = text.shape
    M = visual.shape[1]
    print(f"search B{B} N{N} M{M} D{D} S{S} t=({t_low:.3f},{t_high:.3f}) first={first}", flush=True)
    dev = torch.device("cuda")
    # padded rows exercise the row strides
    tp = np.zeros((B, N, D + text_pad), np.float16)
    tp[:, :, :D] = text
    vp = np.zeros((B, M, D + vis_pad), np.float16)
    vp[:, :, :D] = visual
    tt = torch.from_numpy(tp).to(dev)
    vt = torch.from_numpy(vp).to(dev)
    W = M // S
    scores = torch.full((B, W), float("nan"), dtype=torch.float32, device=dev)
    bits = torch.zeros(W, dtype=torch.uint8, device=dev)
    ws_bytes = kvq.kvq_window_search_workspace(B, N, M, D, S)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    kvq.kvq_window_search(B, N, M, D, tt, tt.stride(0), tt.stride(1), vt, vt.stride(0), vt.stride(1), S,
                          t_low, t_high, first, scores, bits, ws, ws_bytes)
    torch.cuda.synchronize()
    return scores.cpu().numpy().astype(np.float64), bits.cpu().numpy()


def check(kvq, text, visual, S, t_low, t_high, first=True, **pad):
    got_s, got_b = run_search(kvq, text, visual, S, t_low, t_high, first, **pad)
    ref_s, ref_b = search.search(text.astype(np.float64), visual.astype(np.float64), S, t_low, t_high, first)
    assert got_s.shape == ref_s.shape
    err = np.abs(got_s - ref_s).max()
    assert err <= SCORE_TOL, f"score error {err}"
    for i in range(ref_b.size):
        ok = admissible(ref_s[:, i], t_low, t_high, first and i == 0)
        assert ref_b[i] in ok
        assert got_b[i] in ok, (i, got_b[i], sorted(ok), ref_b[i], ref_s[:, i])
    return got_s, got_b


def row_widths(score, t_low, t_high):
    """Widths the decision rule (Sec. 3.2.1) gives for scores within MARGIN
    of `score`: the rule is monotone in the score (2, then 4, then 16), so
    these are the widths between its choices at score - MARGIN and
    score + MARGIN."""
    order = (2, 4, 16)
    lo = order.index(search.choose_bits(score - MARGIN, t_low, t_high))
    hi = order.index(search.choose_bits(score + MARGIN, t_low, t_high))
    return order[lo:hi + 1]


def admissible(scores, t_low, t_high, first_fp16):
    """Widths a window may get (Sec. 3.2.3): the batch vote over every
    combination of the rows' admissible widths; 16 only for a forced-fp16
    first window (Sec. 3.2.2)."""
    if first_fp16:
        return {16}
    per_row = [row_widths(float(s), t_low, t_high) for s in scores]
    return {search.batch_vote(c) for c in itertools.product(*per_row)}


@pytest.mark.parametrize("B,N,M,D,S", [
    (1, 1, 64, 8, 64), (2, 5, 3 * 100 + 17, 64, 100), (3, 70, 8 * 64, 520, 64),
    (1, 64, 4 * 256 + 255, 3584, 256), (5, 17, 6 * 16, 4096, 16), (2, 130, 2 * 200, 128, 200),
])
def test_scores_and_widths(kvq, B, N, M, D, S):
    t_low, t_high = search.thresholds(0.5, 2.0)
    text, vis = workloads.search_tokens(B, N, M, D, S, seed=B * 100 + N)
    _, bits = check(kvq, text, vis, S, t_low, t_high)
    assert bits[0] == 16


def test_row_strides_and_first_window_rule(kvq):
    t_low, t_high = search.thresholds(0.3, 2.0)
    text, vis = workloads.search_tokens(2, 9, 10 * 32, 96, 32, seed=7)
    check(kvq, text, vis, 32, t_low, t_high, first=False, text_pad=8, vis_pad=24)
    check(kvq, text, vis, 32, t_low, t_high, first=True, text_pad=8, vis_pad=24)


def test_zero_rows_and_extreme_thresholds(kvq):
    text, vis = workloads.search_tokens(2, 6, 5 * 64, 64, 64, seed=9)
    text[0, 2] = 0
    vis[1, 70:90] = 0                      # part of window 1 of row 1
    vis[0, 256:320] = 0                    # all of window 4 of row 0
    check(kvq, text, vis, 64, 0.3, 0.7)
    _, b = check(kvq, text, vis, 64, 10.0, 20.0, first=False)   # every score below t_low
    assert b.tolist() == [2] * 5
    _, b = check(kvq, text, vis, 64, -10.0, -5.0, first=False)  # every score above t_high
    assert b.tolist() == [16] * 5


def test_batch_vote(kvq):
    # three rows: row 2's prompt points the other way, so its scores flip
    # sign; the vote follows rows 0 and 1 wherever they agree
    text, vis = workloads.search_tokens(3, 8, 12 * 64, 128, 64, seed=11)
    text[2] = -text[2]
    s, b = check(kvq, text, vis, 64, 0.2, 0.6, first=False)
    assert (s[2] < 0).mean() > 0.9


def test_repeatable(kvq):
    text, vis = workloads.search_tokens(2, 20, 6 * 128, 512, 128, seed=3)
    a = run_search(kvq, text, vis, 128, 0.25, 0.75)
    b = run_search(kvq, text, vis, 128, 0.25, 0.75)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_full_size(kvq):
    # 128 windows of 256 visual tokens and a 64-token prompt, dim 3584 (the
    # hidden size of the pages' Qwen2-VL-7B / LLaVA-OneVision-7B), batch 1
    t_low, t_high = search.thresholds(0.5, 2.0)
    text, vis = workloads.search_tokens(1, 64, 128 * 256, 3584, 256, seed=0)
    _, bits = check(kvq, text, vis, 256, t_low, t_high)
    assert set(bits.tolist()) <= {16, 4, 2} and bits[0] == 16


@pytest.mark.parametrize("side", ["below_low", "above_low", "below_high", "above_high"])
def test_scores_at_thresholds(kvq, side):
    """Thresholds placed a third of the margin from a window's oracle score,
    so that window's admissible set is exactly the two widths next to that
    threshold: a kernel writing the third width fails."""
    text, vis = workloads.search_tokens(1, 16, 9 * 64, 256, 64, seed=21)
    ref, _ = search.search(text.astype(np.float64), vis.astype(np.float64), 64, 0.0, 1.0, False)
    j = int(np.argsort(ref[0])[4])                     # a window in the middle of the range
    s = float(ref[0, j])
    d = MARGIN / 3
    t_low, t_high = {"below_low": (s + d, s + 0.5), "above_low": (s - d, s + 0.5),
                     "below_high": (s - 0.5, s + d), "above_high": (s - 0.5, s - d)}[side]
    _, bits = check(kvq, text, vis, 64, t_low, t_high, first=False)
    near_low = side.endswith("low")
    assert admissible(ref[:, j], t_low, t_high, False) == ({2, 4} if near_low else {4, 16})
    assert bits[j] != (16 if near_low else 2)
