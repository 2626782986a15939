"""Byte layout of packed codes and (scale, zero) pairs (oracle side).

The pages define no storage format; this is the format written down in
``include/kvq.h`` ("Cache layout"), implemented here a second time with plain
NumPy so that the HIP path's bytes can be compared bit for bit.

Code rows (keys, b in {2, 4, 8}): one row of RB = d*b/8 bytes per token; the
code of channel c sits in byte floor(c*b/8) at bit (c*b) mod 8, least
significant bits first.

Code pairs (values): tokens 2p and 2p+1 share a block of 2*RB bytes made of
RB/2 little-endian 32-bit words; word w holds bytes 2w, 2w+1 of token 2p's
row in its low half and the same two bytes of token 2p+1's row in its high
half.  A missing odd token reads as zero bytes here.

Key meta: pair (s16, z16) of group j, channel c at pair index j*d + c.
Value meta: pair of token t, channel group g at pair index
((t//2) * (d/G) + g) * 2 + t%2.
"""
from __future__ import annotations

import numpy as np

__all__ = ["pack_rows", "unpack_rows", "pair_interleave", "pair_deinterleave",
           "pack_values", "unpack_values", "pack_key_meta", "unpack_key_meta",
           "pack_value_meta", "unpack_value_meta"]


def pack_rows(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes uint8 [n][d] -> bytes uint8 [n][d*bits/8] (key row format)."""
    n, d = codes.shape
    per = 8 // bits
    assert (d * bits) % 8 == 0 and codes.max(initial=0) < (1 << bits)
    out = np.zeros((n, d // per), dtype=np.uint8)
    for byte in range(d // per):
        for j in range(per):
            c = byte * per + j
            out[:, byte] |= (codes[:, c].astype(np.uint8) << np.uint8(j * bits)).astype(np.uint8)
    return out


def unpack_rows(rows: np.ndarray, bits: int, d: int) -> np.ndarray:
    """Inverse of pack_rows: bytes [n][d*bits/8] -> codes uint8 [n][d]."""
    n = rows.shape[0]
    per = 8 // bits
    mask = (1 << bits) - 1
    out = np.zeros((n, d), dtype=np.uint8)
    for c in range(d):
        out[:, c] = (rows[:, c // per] >> ((c % per) * bits)) & mask
    return out


def pair_interleave(rows: np.ndarray) -> np.ndarray:
    """Rows [n][RB] -> pair blocks [ceil(n/2)][2*RB] (16-bit interleave)."""
    n, rb = rows.shape
    assert rb % 4 == 0
    npair = (n + 1) // 2
    padded = np.zeros((2 * npair, rb), dtype=np.uint8)
    padded[:n] = rows
    out = np.zeros((npair, 2 * rb), dtype=np.uint8)
    even, odd = padded[0::2], padded[1::2]          # tokens 2p and 2p+1
    for w in range(rb // 2):
        out[:, 4 * w + 0] = even[:, 2 * w]
        out[:, 4 * w + 1] = even[:, 2 * w + 1]
        out[:, 4 * w + 2] = odd[:, 2 * w]
        out[:, 4 * w + 3] = odd[:, 2 * w + 1]
    return out


def pair_deinterleave(blocks: np.ndarray, n: int) -> np.ndarray:
    """Pair blocks [npair][2*RB] -> rows [n][RB]."""
    npair, rb2 = blocks.shape
    rb = rb2 // 2
    rows = np.zeros((2 * npair, rb), dtype=np.uint8)
    for w in range(rb // 2):
        rows[0::2, 2 * w] = blocks[:, 4 * w + 0]
        rows[0::2, 2 * w + 1] = blocks[:, 4 * w + 1]
        rows[1::2, 2 * w] = blocks[:, 4 * w + 2]
        rows[1::2, 2 * w + 1] = blocks[:, 4 * w + 3]
    return rows[:n]


def pack_values(codes: np.ndarray, bits: int) -> np.ndarray:
    """Value codes uint8 [n][d] -> pair blocks [ceil(n/2)][d*bits/4]."""
    return pair_interleave(pack_rows(codes, bits))


def unpack_values(blocks: np.ndarray, bits: int, d: int, n: int) -> np.ndarray:
    return unpack_rows(pair_deinterleave(blocks, n), bits, d)


def pack_key_meta(s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """Key (s, z) [ng][d] fp16 -> fp16 [ng*d*2]: pair j*d + c = (s, z)."""
    ng, d = s16.shape
    out = np.zeros((ng, d, 2), dtype=np.float16)
    out[:, :, 0] = s16
    out[:, :, 1] = z16
    return out.reshape(-1)


def unpack_key_meta(meta: np.ndarray, ng: int, d: int):
    m = meta[: ng * d * 2].reshape(ng, d, 2)
    return m[:, :, 0].copy(), m[:, :, 1].copy()


def pack_value_meta(s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """Value (s, z) [n][ng] fp16 -> fp16 [ceil(n/2)*ng*2*2] (pair layout)."""
    n, ng = s16.shape
    npair = (n + 1) // 2
    out = np.zeros((npair, ng, 2, 2), dtype=np.float16)
    t = np.arange(n)
    out[t // 2, :, t % 2, 0] = s16
    out[t // 2, :, t % 2, 1] = z16
    return out.reshape(-1)


def unpack_value_meta(meta: np.ndarray, n: int, ng: int):
    npair = (n + 1) // 2
    m = meta[: npair * ng * 4].reshape(npair, ng, 2, 2)
    t = np.arange(n)
    return m[t // 2, :, t % 2, 0].copy(), m[t // 2, :, t % 2, 1].copy()
