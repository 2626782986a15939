"""Pins of the oracle's KIVI state machine and decode attention.

* cache part sizes against hand-derived states (tests/golden/kivi_states.json)
  and a closed-form count, over many prefill lengths and decode steps;
* streaming equals bulk: the keys/values quantized step by step are exactly
  the bulk GroupQuant of the same tokens (group locality);
* attention against torch's scaled_dot_product_attention (CPU, float64), a
  library routine: on an all-fp16 cache directly, and on a quantized cache
  after the test itself lines up every token's dequantized key and value.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle.kivi import KiviStream, kivi_lengths
from oracle.quant import quantize_keys, quantize_values, dequantize_keys, dequantize_values

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kivi_states.json")))


def _sdpa(q, k, v, scale):
    """torch SDPA, fp64 CPU; q [g][d], k/v [N][d] shared by all g heads."""
    qt = torch.tensor(np.asarray(q, np.float64))[None, :, None, :]
    g = qt.shape[1]
    kt = torch.tensor(np.asarray(k, np.float64))[None, None].expand(1, g, -1, -1).contiguous()
    vt = torch.tensor(np.asarray(v, np.float64))[None, None].expand(1, g, -1, -1).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o[0, :, 0, :].numpy()


def _stream(l, n_dec, d=32, bits=2, G=32, R=64, seed=0):
    rng = np.random.default_rng(seed)
    n = l + n_dec
    xk = rng.standard_normal((n, d)).astype(np.float16)
    xv = rng.standard_normal((n, d)).astype(np.float16)
    st = KiviStream(d, bits, G, R)
    st.prefill(xk[:l], xv[:l])
    for t in range(l, n):
        st.decode_append(xk[t], xv[t])
    return st, xk, xv


def test_golden_states():
    for case in GOLD["cases"]:
        st, _, _ = _stream(case["L"], 1, d=32, G=case["G"] if case["G"] <= 32 else 32, R=case["R"])
        assert list(st.lengths) == case["state"], case["name"]
        assert list(kivi_lengths(case["L"], 1, case["R"])) == case["state"], case["name"]


@pytest.mark.parametrize("R", [32, 64])
def test_lengths_closed_form_many_steps(R):
    for l in (0, 1, 31, 32, 33, 100, 128, 129):
        st, _, _ = _stream(l, 0, R=R)
        assert st.lengths == kivi_lengths(l, 0, R)
        for step in range(1, 2 * R + 3):
            st.decode_append(np.zeros(32, np.float16), np.zeros(32, np.float16))
            assert st.lengths == kivi_lengths(l, step, R), (l, step)
            n_kq, r_k, n_vq, r_v = st.lengths
            assert r_k < R and r_v <= R and n_kq % R == 0


@pytest.mark.parametrize("l,n_dec", [(0, 200), (70, 130), (256, 1), (300, 77)])
def test_streaming_equals_bulk(l, n_dec):
    st, xk, xv = _stream(l, n_dec, bits=4)
    n_kq, r_k, n_vq, r_v = st.lengths
    total = l + n_dec
    c, s, z = quantize_keys(xk[:n_kq], 4, 32)
    assert np.array_equal(st.kq, c) and np.array_equal(st.ks, s) and np.array_equal(st.kz, z)
    c, s, z = quantize_values(xv[:n_vq], 4, 32)
    assert np.array_equal(st.vq, c) and np.array_equal(st.vs, s) and np.array_equal(st.vz, z)
    assert np.array_equal(st.k_res, xk[n_kq:total]) and np.array_equal(st.v_res, xv[n_vq:total])


def test_all_fp16_reduces_to_textbook_attention():
    # prompt shorter than R: nothing is quantized
    st, xk, xv = _stream(20, 5, R=64)
    assert st.lengths == (0, 25, 0, 25)
    rng = np.random.default_rng(9)
    q = rng.standard_normal((3, 32)).astype(np.float16)
    got = st.attend(q, 0.3)
    ref = _sdpa(q, xk.astype(np.float64), xv.astype(np.float64), 0.3)
    assert np.allclose(got, ref, atol=1e-13, rtol=1e-12)


@pytest.mark.parametrize("l,n_dec", [(256, 1), (191, 40)])
def test_quantized_attention_matches_library_on_aligned_tokens(l, n_dec):
    st, xk, xv = _stream(l, n_dec, bits=2)
    n_kq, r_k, n_vq, r_v = st.lengths
    assert n_kq != n_vq
    total = l + n_dec
    # line every token up with its own key and value, as the cache stores it
    keys = np.zeros((total, 32))
    vals = np.zeros((total, 32))
    keys[:n_kq] = dequantize_keys(st.kq, st.ks, st.kz, 32)
    keys[n_kq:] = st.k_res
    vals[:n_vq] = dequantize_values(st.vq, st.vs, st.vz, 32)
    vals[n_vq:] = st.v_res
    rng = np.random.default_rng(11)
    q = rng.standard_normal((4, 32)).astype(np.float16)
    got = st.attend(q, 1 / np.sqrt(32))
    ref = _sdpa(q, keys, vals, 1 / np.sqrt(32))
    assert np.allclose(got, ref, atol=1e-13, rtol=1e-12)
    # the test has teeth: values shifted by one token give another result
    assert not np.allclose(_sdpa(q, keys, np.roll(vals, 1, axis=0), 1 / np.sqrt(32)), got)


def test_quantization_error_bound_on_output():
    # |l' - l| <= scale * sum_c |q_c| s_c / 2 per token (keys), values move by
    # at most s/2; the output error is bounded accordingly
    st, xk, xv = _stream(512, 1, d=64, bits=4, R=64)
    rng = np.random.default_rng(12)
    q = rng.standard_normal((1, 64)).astype(np.float16)
    scale = 0.125
    got = st.attend(q, scale)
    exact = _sdpa(q, xk.astype(np.float64), xv.astype(np.float64), scale)
    n_kq = st.lengths[0]
    s_k = np.repeat(st.ks.astype(np.float64), 32, axis=0)                # [n_kq][d]
    eps = scale * np.max(np.abs(q.astype(np.float64)) @ (s_k.T / 2)) if n_kq else 0.0
    v_err = np.max(np.repeat(st.vs.astype(np.float64), 32, axis=1)) / 2
    vmax = np.max(np.abs(xv.astype(np.float64))) + v_err
    bound = (np.exp(2 * eps) - 1) * vmax + v_err
    assert np.max(np.abs(got - exact)) <= bound
