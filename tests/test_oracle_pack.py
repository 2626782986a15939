"""Pins of the oracle's byte layout: hand-derived bytes from the written
definition in include/kvq.h (the pages define no layout) and round trips."""
import json
import os

import numpy as np
import pytest

from oracle import pack

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pack_examples.json")))


def test_rows_golden():
    for ex in GOLD["rows"]:
        got = pack.pack_rows(np.array(ex["codes"], dtype=np.uint8), ex["bits"])
        assert got.tolist() == ex["bytes"], ex["why"]


def test_pairs_golden():
    for ex in GOLD["pairs"]:
        got = pack.pair_interleave(np.array(ex["rows"], dtype=np.uint8))
        assert got.tolist() == ex["blocks"], ex["why"]


def test_meta_golden():
    km = GOLD["key_meta"]
    got = pack.pack_key_meta(np.array(km["s"], np.float16), np.array(km["z"], np.float16))
    assert got.tolist() == km["flat"]
    vm = GOLD["value_meta"]
    got = pack.pack_value_meta(np.array(vm["s"], np.float16), np.array(vm["z"], np.float16))
    assert got.tolist() == vm["flat"], vm["why"]


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [1, 2, 7, 64])
def test_round_trips(bits, d, n):
    rng = np.random.default_rng([bits, d, n])
    codes = rng.integers(0, 1 << bits, size=(n, d)).astype(np.uint8)
    rows = pack.pack_rows(codes, bits)
    assert rows.shape == (n, d * bits // 8)
    assert np.array_equal(pack.unpack_rows(rows, bits, d), codes)
    blocks = pack.pack_values(codes, bits)
    assert blocks.shape == ((n + 1) // 2, d * bits // 4)
    assert np.array_equal(pack.unpack_values(blocks, bits, d, n), codes)
    ng = d // 32
    s = rng.standard_normal((n, ng)).astype(np.float16)
    z = rng.standard_normal((n, ng)).astype(np.float16)
    s2, z2 = pack.unpack_value_meta(pack.pack_value_meta(s, z), n, ng)
    assert np.array_equal(s, s2) and np.array_equal(z, z2)
    ks = rng.standard_normal((3, d)).astype(np.float16)
    kz = rng.standard_normal((3, d)).astype(np.float16)
    ks2, kz2 = pack.unpack_key_meta(pack.pack_key_meta(ks, kz), 3, d)
    assert np.array_equal(ks, ks2) and np.array_equal(kz, kz2)


def test_channel_bit_position_brute_force():
    # every single-channel code lands at byte c*b//8, bit (c*b)%8
    for bits in (2, 4, 8):
        for c in range(16):
            codes = np.zeros((1, 16), np.uint8)
            codes[0, c] = (1 << bits) - 1
            row = pack.pack_rows(codes, bits)[0]
            expect = np.zeros(16 * bits // 8, np.uint8)
            expect[c * bits // 8] = ((1 << bits) - 1) << ((c * bits) % 8)
            assert np.array_equal(row, expect)
