"""Pins of the oracle's WindowQuant reorder (Sec. 3.3.1-3.3.2).

* the permutation against Python's stable sort and, on tiny inputs, against
  brute-force enumeration of every permutation;
* hand-derived segment tables and gather lists (tests/golden);
* permutation invariance (Eq. 12-13): the reordered cache gives the same
  output as the same windows quantized in place, in token order;
* all-fp16 windows reduce to torch's scaled_dot_product_attention;
* the mixed-precision workload's window bit assignment against a
  hand-derived example that each plausible slip of its rule fails.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import windows

GOLD_DIR = os.path.join(os.path.dirname(__file__), "golden")

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "window_examples.json")))


def test_golden_tables():
    for case in GOLD["cases"]:
        assert windows.reorder(case["win_bits"]) == case["perm"]
        segs = windows.segment_table(case["win_bits"], case["S"], case["d"], case["G"])
        assert [list(s) for s in segs] == case["segments"], case["why"]
    g = GOLD["gather"]
    assert windows.row_gather(g["perm"], g["S"]).tolist() == g["rows"]


def test_reorder_brute_force_tiny():
    rng = np.random.default_rng(0)
    for trial in range(40):
        w = int(rng.integers(1, 7))
        bits = [int(b) for b in rng.choice([16, 8, 4, 2], size=w)]
        ok = [p for p in itertools.permutations(range(w))
              if all(bits[p[i]] > bits[p[i + 1]] or (bits[p[i]] == bits[p[i + 1]] and p[i] < p[i + 1])
                     for i in range(w - 1))]
        assert len(ok) == 1
        assert windows.reorder(bits) == list(ok[0])


def test_reorder_matches_stable_sort_large():
    rng = np.random.default_rng(1)
    bits = rng.choice([8, 4, 2], size=128)
    perm = windows.reorder(bits)
    assert perm == sorted(range(128), key=lambda i: -int(bits[i]))   # Python sort is stable
    segs = windows.segment_table(bits, 256, 128, 32)
    assert sum(s.n_tok for s in segs) == 128 * 256
    assert [s.bits for s in segs] == [b for b in (8, 4, 2) if b in set(bits.tolist())]


@pytest.mark.parametrize("G", [32, 64])
def test_permutation_invariance(G):
    rng = np.random.default_rng(2)
    W, S, d = 6, 64, 64
    n = W * S + 9
    xk = rng.standard_normal((n, d)).astype(np.float16)
    xv = rng.standard_normal((n, d)).astype(np.float16)
    bits = [2, 8, 4, 2, 16, 4]
    q = rng.standard_normal((3, d)).astype(np.float16)
    st = windows.WindowStream(xk, xv, bits, S, G)
    a = st.attend(q, 0.125)
    b = windows.attend_in_place(xk, xv, bits, S, G, q, 0.125)
    assert np.allclose(a, b, atol=1e-13, rtol=1e-12)
    # and the quantized data really is different from fp16 (the test has teeth)
    assert not np.allclose(a, windows.attend_in_place(xk, xv, [16] * W, S, G, q, 0.125), atol=1e-6)


def test_all_fp16_windows_is_textbook_attention():
    rng = np.random.default_rng(3)
    W, S, d = 4, 32, 64
    n = W * S + 5
    xk = rng.standard_normal((n, d)).astype(np.float16)
    xv = rng.standard_normal((n, d)).astype(np.float16)
    q = rng.standard_normal((2, d)).astype(np.float16)
    st = windows.WindowStream(xk, xv, [16] * W, S, 32)
    got = st.attend(q, 0.2)
    qt = torch.tensor(q.astype(np.float64))[None, :, None, :]
    kt = torch.tensor(xk.astype(np.float64))[None, None].expand(1, 2, -1, -1).contiguous()
    vt = torch.tensor(xv.astype(np.float64))[None, None].expand(1, 2, -1, -1).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.2)[0, :, 0].numpy()
    assert np.allclose(got, ref, atol=1e-13, rtol=1e-12)


def test_workload_window_bits_mix():
    w = workloads.get("qwen2_7b_windows").scaled(windows=20, text_tokens=8)
    k = np.stack([workloads.unit_kv(w, 0, h, n_tokens=w.windows * w.window_tokens + 8)[0]
                  for h in range(w.n_kv_heads)])[None]
    bits = workloads.window_bits(w, k)
    assert sorted(bits.tolist()).count(8) == 2 and sorted(bits.tolist()).count(4) == 6
    full = workloads.get("qwen2_7b_windows")
    assert int(np.floor(full.frac8 * 128)) == 12 and int(np.floor((full.frac8 + full.frac4) * 128)) == 51


def _pin_keys(e):
    """Keys [1][Hkv][N][d] of the hand-derived window-bits example: each
    window's two tokens (and the two text tokens) are mean + e and mean - e."""
    H, d, S = e["n_kv_heads"], e["d_h"], e["window_tokens"]
    means = [np.array(m, dtype=np.float64) for m in e["window_means"]] + [np.array(e["text_mean"], np.float64)]
    off = np.array(e["token_offsets"], dtype=np.float64)          # [Hkv][d]
    k = np.zeros((1, H, len(means) * S, d), dtype=np.float64)
    for i, m in enumerate(means):
        k[0, :, i * S] = m + off
        k[0, :, i * S + 1] = m - off
    assert np.array_equal(k.astype(np.float16).astype(np.float64), k)   # exact in fp16
    return k.astype(np.float16)


def _pin_workload(e):
    W = len(e["window_means"])
    return workloads.get("qwen2_7b_windows").scaled(
        n_q_heads=e["n_kv_heads"], n_kv_heads=e["n_kv_heads"], d_h=e["d_h"], windows=W,
        window_tokens=e["window_tokens"], text_tokens=e["text_tokens"],
        context=W * e["window_tokens"] + e["text_tokens"] - 1, frac8=e["frac8"], frac4=e["frac4"])


def test_window_bits_hand_derived_example():
    """workloads.window_bits against a hand-derived assignment (golden file):
    concatenated-head means, descending cosine, ties to the lower index."""
    e = json.load(open(os.path.join(GOLD_DIR, "window_bits_example.json")))
    w = _pin_workload(e)
    bits = workloads.window_bits(w, _pin_keys(e))
    assert bits.tolist() == e["bits"]


def test_window_bits_example_rejects_plausible_slips():
    """The example tells apart the rule from each plausible slip: ranking by
    ascending cosine, dropping kv heads from the concatenated mean, averaging
    per-head cosines, and breaking ties to the higher index.  Each slip is
    planted here (on the CPU) and must give its hand-derived, different
    answer."""
    e = json.load(open(os.path.join(GOLD_DIR, "window_bits_example.json")))
    w = _pin_workload(e)
    k = _pin_keys(e)[0].astype(np.float64)                          # [Hkv][N][d]
    H, W, S = w.n_kv_heads, w.windows, w.window_tokens
    win = k[:, :W * S].reshape(H, W, S, w.d_h).mean(axis=2)         # [Hkv][W][d]
    txt = k[:, W * S:].mean(axis=1)                                 # [Hkv][d]

    def cos(a, b):
        return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))

    def assign(score, descending=True, lower_first=True):
        key = (lambda i: ((-score[i] if descending else score[i]), i if lower_first else -i))
        order = sorted(range(W), key=key)
        n8, n84 = int(np.floor(w.frac8 * W)), int(np.floor((w.frac8 + w.frac4) * W))
        out = [2] * W
        for r, i in enumerate(order):
            out[i] = 8 if r < n8 else (4 if r < n84 else 2)
        return out

    concat = [cos(win[:, i].reshape(-1), txt.reshape(-1)) for i in range(W)]
    assert np.allclose(concat, e["cosines"], rtol=0, atol=1e-12)
    assert assign(concat) == e["bits"]
    wrong = e["wrong_rules"]
    assert assign(concat, descending=False) == wrong["ascending_rank"]
    assert assign([cos(win[0, i], txt[0]) for i in range(W)]) == wrong["first_head_only"]
    assert assign([np.mean([cos(win[h, i], txt[h]) for h in range(H)]) for i in range(W)]) == \
        wrong["mean_of_per_head_cosines"]
    assert assign(concat, lower_first=False) == wrong["ties_to_higher_index"]
    for name, bits in wrong.items():
        assert bits != e["bits"], name
