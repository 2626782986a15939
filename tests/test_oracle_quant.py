"""Pins of the oracle's quantizer against what the pages fix.

* worked examples derived by hand from the formula (tests/golden);
* brute force: the code is the nearest of the 2^b levels q*s+z (except ties);
* the per-element error bound s/2 for round-to-nearest;
* every non-constant group reaches code 0 and code 2^b-1;
* the grouping axes: a key outlier channel leaves the other channels alone,
  a changed value token leaves the other tokens alone (KIVI note, "Key cache
  quantization dimension" / "Value cache quantization dimension").
"""
import json
import os

import numpy as np
import pytest

from oracle.quant import (quantize_groups, quantize_keys, quantize_values,
                          dequantize_keys, dequantize_values)

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _groups(rng, n, g, kind):
    if kind == "normal":
        x = rng.standard_normal((n, g))
    elif kind == "outlier":
        x = rng.standard_normal((n, g)) * 8.0
        x[:, 0] *= 10
    elif kind == "tiny":
        x = rng.standard_normal((n, g)) * 1e-3
    elif kind == "ties":
        x = rng.integers(-8, 8, size=(n, g)) * 0.5
    else:
        raise ValueError(kind)
    return x.astype(np.float16)


def test_worked_examples():
    data = json.load(open(os.path.join(GOLD, "quant_examples.json")))
    for ex in data["examples"]:
        x = np.array(ex["x"], dtype=np.float16)[None, :]
        codes, s16, z16 = quantize_groups(x, ex["bits"])
        assert codes[0].tolist() == ex["codes"], ex["why"]
        # compare bit patterns: the sign of a zero matters
        assert s16[:1].view(np.uint16)[0] == np.float16(ex["s16"]).view(np.uint16), ex["why"]
        assert z16[:1].view(np.uint16)[0] == np.float16(ex["z16"]).view(np.uint16), ex["why"]


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("kind", ["normal", "outlier", "tiny", "ties"])
def test_brute_force_nearest_level(bits, kind):
    rng = np.random.default_rng([bits, len(kind)])
    x = _groups(rng, 2000, 32, kind)
    codes, s16, z16 = quantize_groups(x, bits)
    s = s16.astype(np.float64)[:, None, None]
    z = z16.astype(np.float64)[:, None, None]
    levels = np.arange(1 << bits, dtype=np.float64)[None, None, :] * s + z
    dist = np.abs(x.astype(np.float64)[:, :, None] - levels)        # [n][G][levels]
    best = dist.min(axis=2)
    mine = np.take_along_axis(dist, codes[:, :, None].astype(np.int64), axis=2)[:, :, 0]
    # any disagreement must be an exact tie up to fp32 rounding of (x - z) / s
    gap = mine - best
    tol = 1e-6 * np.maximum(s[:, :, 0], 1e-30) + 1e-12
    assert np.all(gap <= tol), float(gap.max())
    # zero-range groups code everything as 0
    assert np.all(codes[s16 == 0] == 0)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_error_bound_half_scale(bits):
    rng = np.random.default_rng(bits)
    x = _groups(rng, 4000, 32, "normal")
    codes, s16, z16 = quantize_groups(x, bits)
    xr = codes.astype(np.float64) * s16.astype(np.float64)[:, None] + z16.astype(np.float64)[:, None]
    err = np.abs(xr - x.astype(np.float64))
    normal = s16.astype(np.float64) >= 2.0 ** -14
    bound = s16.astype(np.float64)[:, None] / 2 * (1 + 1e-3)
    assert np.all(err[normal] <= np.broadcast_to(bound, err.shape)[normal])


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_group_extrema_reach_both_ends(bits):
    rng = np.random.default_rng(10 + bits)
    x = _groups(rng, 3000, 32, "outlier")
    codes, s16, _ = quantize_groups(x, bits)
    live = s16 > 0
    xa = x.astype(np.float32)
    at_min = codes[np.arange(len(x)), xa.argmin(1)]
    at_max = codes[np.arange(len(x)), xa.argmax(1)]
    assert np.all(at_min[live] == 0)
    assert np.all(at_max[live] == (1 << bits) - 1)
    # the zero point is the group minimum, exactly
    assert np.array_equal(quantize_groups(x, bits)[2], x.min(axis=1))


def test_key_groups_are_per_channel_over_G_tokens():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((64, 16)).astype(np.float16)
    codes, s, z = quantize_keys(k, 2, 32)
    assert codes.shape == (64, 16) and s.shape == (2, 16)
    k2 = k.copy()
    k2[:, 5] *= np.float16(200)                       # an outlier channel
    codes2, s2, z2 = quantize_keys(k2, 2, 32)
    other = [c for c in range(16) if c != 5]
    assert np.array_equal(codes[:, other], codes2[:, other])
    assert np.array_equal(s[:, other], s2[:, other])
    # a change in tokens 32..63 leaves group 0 (tokens 0..31) alone
    k3 = k.copy()
    k3[40] += np.float16(3)
    codes3, s3, _ = quantize_keys(k3, 2, 32)
    assert np.array_equal(codes3[:32], codes[:32]) and np.array_equal(s3[0], s[0])
    # group 0 of channel c is exactly the group of tokens 0..31 of that channel
    c0, s0, z0 = quantize_groups(np.ascontiguousarray(k[:32, 7])[None, :], 2)
    assert np.array_equal(codes[:32, 7], c0[0]) and s[0, 7] == s0[0] and z[0, 7] == z0[0]


def test_value_groups_are_per_token_over_G_channels():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((10, 64)).astype(np.float16)
    codes, s, z = quantize_values(v, 4, 32)
    assert codes.shape == (10, 64) and s.shape == (10, 2)
    v2 = v.copy()
    v2[6] *= np.float16(50)
    codes2, s2, _ = quantize_values(v2, 4, 32)
    other = [t for t in range(10) if t != 6]
    assert np.array_equal(codes[other], codes2[other]) and np.array_equal(s[other], s2[other])
    # group 1 of token 3 is channels 32..63 of that token
    c1, s1, z1 = quantize_groups(v[3:4, 32:64], 4)
    assert np.array_equal(codes[3, 32:], c1[0]) and s[3, 1] == s1[0] and z[3, 1] == z1[0]
    # a constant group has scale 0 and dequantizes exactly
    v3 = v.copy()
    v3[0, :32] = np.float16(0.75)
    c3, s3, z3 = quantize_values(v3, 2, 32)
    assert s3[0, 0] == 0 and np.all(dequantize_values(c3, s3, z3, 32)[0, :32] == 0.75)


def test_dequantize_matches_formula_elementwise():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((32, 8)).astype(np.float16)
    codes, s, z = quantize_keys(k, 4, 32)
    deq = dequantize_keys(codes, s, z, 32)
    for t in (0, 17, 31):
        for c in (0, 3, 7):
            assert deq[t, c] == float(codes[t, c]) * float(s[0, c]) + float(z[0, c])


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_dequantize_round_trip_groups_with_different_ranges(bits):
    # groups of very different ranges: a wrong group-to-scale mapping in the
    # dequantizer would blow the s/2 bound by orders of magnitude
    rng = np.random.default_rng(20 + bits)
    v = rng.standard_normal((6, 128)).astype(np.float32)
    v *= np.array([100.0, 0.01, 3.0, 0.3], np.float32).repeat(32)[None, :]
    v = v.astype(np.float16)
    c, s, z = quantize_values(v, bits, 32)
    err = np.abs(dequantize_values(c, s, z, 32) - v.astype(np.float64))
    for g in range(4):
        assert err[:, 32 * g:32 * (g + 1)].max() <= s[:, g].astype(np.float64).max() / 2 * 1.001
    k = rng.standard_normal((64, 16)).astype(np.float32)
    k[:32] *= 100.0
    k[32:] *= 0.01
    k = k.astype(np.float16)
    c, s, z = quantize_keys(k, bits, 32)
    err = np.abs(dequantize_keys(c, s, z, 32) - k.astype(np.float64))
    assert err[32:].max() <= s[1].astype(np.float64).max() / 2 * 1.001
    assert err[:32].max() <= s[0].astype(np.float64).max() / 2 * 1.001
