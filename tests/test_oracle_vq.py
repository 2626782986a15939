"""Pins of the VQ (codebook) decode-attention oracle (oracle/vq.py) against
what the VQ-LLM note fixes and the mathematics gives: a hand-derived example
(tests/golden/vq_examples.json: lookups, residual rounds, concatenation,
and the attention weights 1/2-1/2 of a zero query and 3/4-1/4 of logits
ln 3 apart), codebooks whose entries encode their own (group, entry) index
(catches a transposed or shifted lookup), residual rounds adding, the closed
form of identical keys (the mean of the values), a single token, and torch's
scaled_dot_product_attention (CPU, float64) over the dequantized cache."""
import json
import os

import numpy as np
import torch

from oracle import vq

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "vq_examples.json")


def test_hand_derived_example():
    g = json.load(open(GOLDEN))
    books = np.array(g["books"], dtype=np.float64)
    codes = np.array(g["codes"], dtype=np.uint8)
    assert np.array_equal(vq.dequantize(codes, books), np.array(g["rows"], dtype=np.float64))
    for qk, ok in (("q_zero", "out_zero"), ("q_ln3", "out_ln3")):
        out = vq.vq_attention(np.array([g[qk]]), codes, codes, books, books, 1.0)
        assert np.allclose(out[0], g[ok], rtol=0, atol=1e-12), (qk, out[0])


def test_entries_name_their_group_and_index():
    # entry e of sub-space j in round 0 is (e, j, 7, -e): a lookup from the
    # wrong sub-space, a transposed code array or a shifted channel shows
    R, G, E = 1, 5, 256
    books = np.zeros((R, G, E, 4))
    for j in range(G):
        for e in range(E):
            books[0, j, e] = (e, j, 7, -e)
    rng = np.random.default_rng(3)
    codes = rng.integers(0, E, size=(9, R, G)).astype(np.uint8)
    rows = vq.dequantize(codes, books)
    assert rows.shape == (9, 4 * G)
    for t in range(9):
        for j in range(G):
            assert rows[t, 4 * j:4 * j + 4].tolist() == [codes[t, 0, j], j, 7, -int(codes[t, 0, j])]


def test_residual_rounds_add():
    rng = np.random.default_rng(4)
    books = rng.standard_normal((2, 8, 256, 4))
    codes = rng.integers(0, 256, size=(50, 2, 8)).astype(np.uint8)
    both = vq.dequantize(codes, books)
    r0 = vq.dequantize(codes[:, :1], books[:1])
    r1 = vq.dequantize(codes[:, 1:], books[1:])
    assert np.allclose(both, r0 + r1, rtol=0, atol=1e-12)


def test_identical_keys_average_the_values():
    rng = np.random.default_rng(5)
    kb = rng.standard_normal((1, 16, 256, 4))
    vb = rng.standard_normal((1, 16, 256, 4))
    kc = np.tile(rng.integers(0, 256, size=(1, 1, 16)), (40, 1, 1)).astype(np.uint8)
    vc = rng.integers(0, 256, size=(40, 1, 16)).astype(np.uint8)
    q = rng.standard_normal((3, 64))
    out = vq.vq_attention(q, kc, vc, kb, vb, 0.125)
    mean = vq.dequantize(vc, vb).mean(axis=0)
    assert np.allclose(out, np.tile(mean, (3, 1)), rtol=0, atol=1e-12)


def test_single_token_returns_its_value():
    rng = np.random.default_rng(6)
    kb, vb = rng.standard_normal((2, 2, 32, 256, 4))           # two rounds, 32 sub-spaces each
    kc = rng.integers(0, 256, size=(1, 2, 32)).astype(np.uint8)
    vc = rng.integers(0, 256, size=(1, 2, 32)).astype(np.uint8)
    out = vq.vq_attention(rng.standard_normal((2, 128)), kc, vc, kb, vb, 0.1)
    assert np.allclose(out, np.tile(vq.dequantize(vc, vb)[0], (2, 1)), rtol=0, atol=1e-12)


def test_attention_matches_sdpa():
    rng = np.random.default_rng(7)
    R, G, n = 2, 32, 300
    kb = rng.standard_normal((R, G, 256, 4))
    vb = rng.standard_normal((R, G, 256, 4))
    kc = rng.integers(0, 256, size=(n, R, G)).astype(np.uint8)
    vc = rng.integers(0, 256, size=(n, R, G)).astype(np.uint8)
    q = rng.standard_normal((4, 4 * G))
    out = vq.vq_attention(q, kc, vc, kb, vb, 1 / np.sqrt(4 * G))
    k = torch.from_numpy(vq.dequantize(kc, kb))[None, None]
    v = torch.from_numpy(vq.dequantize(vc, vb))[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q)[None, :, None, :],
                                                           k.expand(1, 4, n, 4 * G), v.expand(1, 4, n, 4 * G),
                                                           scale=1 / np.sqrt(4 * G))
    assert np.allclose(out, ref[0, :, 0].numpy(), rtol=1e-10, atol=1e-12)
