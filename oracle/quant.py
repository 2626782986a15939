"""Asymmetric round-to-nearest group quantizer (oracle).

Formula (KIVI note, quick read "How it works" and background "Preliminary
study of KV-cache quantization"):  Q(X) = round((X - z) / s),  X' = Q * s + z.

The pages leave s and z implicit; the reading taken (WindowQuant Sec. 3.3.3,
Eq. 16, with unsigned codes q_min = 0, q_max = 2^b - 1):

    s = (max - min) / (2^b - 1)        z = min

with these further readings where the pages are silent:

* s and z are stored as fp16; codes are computed with the *stored* fp16 s and
  z, so the encoder and the decoder use the same numbers;
* rounding is round-half-even (the pages only say "nearest");
* codes are clamped to [0, 2^b - 1] (WindowQuant Eq. 14 clamps);
* a group whose fp16 scale is 0 gets all codes 0 (it dequantizes to z);
* zero extrema are taken as +0 (min + 0 and max + 0 in fp32): the minimum
  of {-0, +0} is not ordered, and z and s each need a single encoding.

Arithmetic is IEEE fp32: fp16 inputs are widened exactly, the range and the
division are single fp32 operations, nothing is fused.

Grouping axes (KIVI note, "Method details" and Algorithm 1):

* keys are quantized per channel: each channel's values over G consecutive
  tokens form one group (GroupQuant(X_K, dim='channel', numGroup=l//G));
* values are quantized per token: each token's d channels are split into
  d/G groups of G consecutive channels (GroupQuant(X_V, dim='token',
  numGroup=d//G)).
"""
from __future__ import annotations

import numpy as np

__all__ = ["quantize_groups", "quantize_keys", "quantize_values",
           "dequantize_keys", "dequantize_values"]


def quantize_groups(x: np.ndarray, bits: int):
    """Quantize along the last axis; every slice x[..., :] is one group.

    x: fp16 array [..., n].  Returns (codes uint8 [..., n], s16 fp16 [...],
    z16 fp16 [...]).
    """
    assert x.dtype == np.float16 and bits in (2, 4, 8)
    qmax = (1 << bits) - 1
    x32 = x.astype(np.float32)
    mn = x32.min(axis=-1) + np.float32(0)        # -0 -> +0
    mx = x32.max(axis=-1) + np.float32(0)        # -0 -> +0
    s32 = (mx - mn) / np.float32(qmax)           # fp32 subtract, fp32 divide
    s16 = s32.astype(np.float16)                 # round to nearest even
    z16 = mn.astype(np.float16)                  # exact: mn is an fp16 value
    s = s16.astype(np.float32)[..., None]
    z = z16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (x32 - z) / s                        # fp32 subtract, fp32 divide
        q = np.rint(t)                           # half-even
        q = np.clip(q, 0, qmax)
    q = np.where(s == 0, np.float32(0), q)
    return q.astype(np.uint8), s16, z16


def quantize_keys(xk: np.ndarray, bits: int, group: int):
    """Per-channel key quantization of n tokens, n % group == 0.

    xk: fp16 [n][d].  Returns codes uint8 [n][d], s16/z16 fp16 [n/group][d]
    (one (s, z) per channel per group of ``group`` tokens).
    """
    n, d = xk.shape
    assert n % group == 0
    g = xk.reshape(n // group, group, d).transpose(0, 2, 1)     # [ng][d][G]
    codes, s16, z16 = quantize_groups(np.ascontiguousarray(g), bits)
    codes = codes.transpose(0, 2, 1).reshape(n, d)
    return codes, s16, z16


def quantize_values(xv: np.ndarray, bits: int, group: int):
    """Per-token value quantization, d % group == 0.

    xv: fp16 [n][d].  Returns codes uint8 [n][d], s16/z16 fp16 [n][d/group].
    """
    n, d = xv.shape
    assert d % group == 0
    codes, s16, z16 = quantize_groups(xv.reshape(n, d // group, group), bits)
    return codes.reshape(n, d), s16, z16


def dequantize_keys(codes, s16, z16, group: int) -> np.ndarray:
    """X' = Q * s + z in float64 for per-channel key groups -> [n][d]."""
    n, d = codes.shape
    s = np.repeat(s16.astype(np.float64), group, axis=0)
    z = np.repeat(z16.astype(np.float64), group, axis=0)
    return codes.astype(np.float64) * s + z


def dequantize_values(codes, s16, z16, group: int) -> np.ndarray:
    """X' = Q * s + z in float64 for per-token value groups -> [n][d]."""
    s = np.repeat(s16.astype(np.float64), group, axis=1)
    z = np.repeat(z16.astype(np.float64), group, axis=1)
    return codes.astype(np.float64) * s + z
