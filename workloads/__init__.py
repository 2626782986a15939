"""Seeded synthetic workloads for low-bit-KV decode attention.

This module is the one place where test and benchmark inputs are made.  Both
the CPU oracle (``oracle/``) and the HIP path (``decode_attention_kivi_amd``)
receive their inputs from here; it holds none of the quantization or attention
arithmetic, only shapes and random draws.

Shapes follow the pages' workloads:

* KIVI (papercache note on arXiv 2402.02750, "Experimental setup"): group size
  G=32, residual length R=128 (some runs R=32); Llama-2-7B attention is
  32 heads x d_h=128 (also the VQ-LLM note's micro-benchmark shape).
* KIVI note, "Key cache quantization dimension": keys carry large outliers on
  a few fixed channels, so keys get fixed outlier channels scaled up.
* PQCache note, "Background": grouped-query attention keeps h_kv < h KV heads.
* WindowQuant (ACM TACO), Section 3.1 / Eq. 4-7: M = T x K visual tokens cut
  into windows of S tokens, followed by the text tokens, which stay fp16.

Recipe (all configs):

* every (batch b, kv head h) stream draws its own keys and values from
  ``numpy.random.default_rng([seed, 0, b, h])``: K then V, each
  ``standard_normal((N, d_h), float32)``, N = context + 1 (the prefilled
  context plus the token of the measured decode step);
* the outlier channels of kv head h come from
  ``default_rng([seed, 2, h]).choice(d_h, n_out, replace=False)`` (sorted);
  those key channels are multiplied by the outlier factor in fp32;
* values are N(0, 1) unless a case scales them (``value_scale``) or gives
  them outlier channels of their own (``default_rng([seed, 3, h])``, same
  draw as the keys'), again in fp32 before the cast;
* queries of batch row b come from ``default_rng([seed, 1, b])``:
  ``standard_normal((Hq, d_h), float32)``;
* everything is then rounded to fp16 (round-to-nearest-even).

Per-stream generators let a test rebuild one (b, h) stream of a full-size
config without drawing the whole tensor.

The mixed-precision config assigns window bit widths by the rule that the
workload names: windows ranked by cosine(mean window key, mean text key) with
the key rows of all kv heads concatenated; the top 10 % get 8 bits, the next
30 % 4 bits, the rest 2 bits; ties go to the lower window index.  That
assignment is an input of the reorder step, so it is made here, in float64.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Iterable, Optional, Tuple

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get", "unit_kv", "queries", "outlier_channels",
    "full_kv", "window_bits", "sample_units", "search_tokens", "ragged_contexts", "pq_inputs", "vq_inputs",
]


@dataclass(frozen=True)
class Workload:
    """One synthetic decode-step workload.

    ``context`` is the number of tokens already cached before the measured
    decode step; the step appends token ``context`` and attends to
    ``context + 1`` tokens.
    """
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    d_h: int
    context: int
    group: int
    residual: int
    bits: int                      # 2/4/8 for uniform KIVI caches, 0 = mixed windows
    n_outlier: int = 0
    outlier_factor: float = 1.0
    windows: int = 0               # number of visual windows (mixed precision)
    window_tokens: int = 0         # S
    text_tokens: int = 0           # fp16 text tokens after the visual windows
    frac8: float = 0.0
    frac4: float = 0.0
    value_scale: float = 1.0       # values drawn N(0, value_scale^2)
    n_value_outlier: int = 0       # value channels per kv head scaled by value_outlier_factor
    value_outlier_factor: float = 1.0
    seed: int = 0
    note: str = ""

    @property
    def n_tokens(self) -> int:
        """Tokens attended by the measured decode step (context + new token)."""
        return self.context + 1

    @property
    def gqa(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def sm_scale(self) -> float:
        return float(1.0 / np.sqrt(self.d_h))

    @property
    def mixed(self) -> bool:
        return self.windows > 0

    def scaled(self, **kw) -> "Workload":
        """A copy with some fields replaced (used for small parity cases)."""
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


def _pct(n: int, frac: float) -> int:
    return int(round(n * frac))


WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("tiny", batch=1, n_q_heads=4, n_kv_heads=4, d_h=64, context=256,
                 group=32, residual=32, bits=2, n_outlier=4, outlier_factor=10.0,
                 note="batch 1, 4 heads MHA, d_h 64, context 256, G32 R32 int2"),
        Workload("llama2_7b", batch=16, n_q_heads=32, n_kv_heads=32, d_h=128,
                 context=4096, group=32, residual=128, bits=2,
                 n_outlier=_pct(128, 0.02), outlier_factor=8.0,
                 note="Llama-2-7B-shaped decode layer, batch 16, context 4096, G32 R128 int2"),
        Workload("llama2_7b_b64_int2", batch=64, n_q_heads=32, n_kv_heads=32, d_h=128,
                 context=2048, group=32, residual=128, bits=2,
                 n_outlier=_pct(128, 0.02), outlier_factor=8.0,
                 note="Llama-2-7B-shaped high batch, batch 64, context 2048, int2"),
        Workload("llama2_7b_b64_int4", batch=64, n_q_heads=32, n_kv_heads=32, d_h=128,
                 context=2048, group=32, residual=128, bits=4,
                 n_outlier=_pct(128, 0.02), outlier_factor=8.0,
                 note="Llama-2-7B-shaped high batch, batch 64, context 2048, int4"),
        Workload("llama31_8b_gqa", batch=4, n_q_heads=32, n_kv_heads=8, d_h=128,
                 context=32768, group=64, residual=128, bits=2,
                 n_outlier=_pct(128, 0.02), outlier_factor=8.0,
                 note="Llama-3.1-8B-shaped GQA long context, batch 4, 32q/8kv, context 32768, G64 R128 int2"),
        Workload("qwen2_7b_windows", batch=1, n_q_heads=28, n_kv_heads=4, d_h=128,
                 context=128 * 256 + 64, group=32, residual=128, bits=0,
                 windows=128, window_tokens=256, text_tokens=64, frac8=0.1, frac4=0.3,
                 note="WindowQuant-style Qwen2-7B-shaped, 128 windows x 256 visual tokens + 64 fp16 text, 8/4/2-bit windows"),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def outlier_channels(w: Workload, h: int) -> np.ndarray:
    """Sorted outlier key channels of kv head ``h``."""
    if w.n_outlier <= 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.default_rng([w.seed, 2, h])
    return np.sort(rng.choice(w.d_h, size=w.n_outlier, replace=False))


def unit_kv(w: Workload, b: int, h: int, n_tokens: Optional[int] = None
            ) -> Tuple[np.ndarray, np.ndarray]:
    """Keys and values of stream (b, h): two fp16 arrays [N][d_h]."""
    n = w.n_tokens if n_tokens is None else n_tokens
    rng = np.random.default_rng([w.seed, 0, b, h])
    k = rng.standard_normal((n, w.d_h), dtype=np.float32)
    v = rng.standard_normal((n, w.d_h), dtype=np.float32)
    oc = outlier_channels(w, h)
    if oc.size:
        k[:, oc] *= np.float32(w.outlier_factor)
    if w.value_scale != 1.0:
        v *= np.float32(w.value_scale)
    if w.n_value_outlier > 0:
        vc = np.sort(np.random.default_rng([w.seed, 3, h]).choice(w.d_h, size=w.n_value_outlier, replace=False))
        v[:, vc] *= np.float32(w.value_outlier_factor)
    return k.astype(np.float16), v.astype(np.float16)


def queries(w: Workload) -> np.ndarray:
    """Decode-step queries, fp16 [B][Hq][d_h]."""
    q = np.empty((w.batch, w.n_q_heads, w.d_h), dtype=np.float16)
    for b in range(w.batch):
        rng = np.random.default_rng([w.seed, 1, b])
        q[b] = rng.standard_normal((w.n_q_heads, w.d_h), dtype=np.float32).astype(np.float16)
    return q


def full_kv(w: Workload, units: Optional[Iterable[Tuple[int, int]]] = None
            ) -> Tuple[np.ndarray, np.ndarray]:
    """Keys and values of every stream, fp16 [B][Hkv][N][d_h] each."""
    shape = (w.batch, w.n_kv_heads, w.n_tokens, w.d_h)
    k = np.empty(shape, dtype=np.float16)
    v = np.empty(shape, dtype=np.float16)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            k[b, h], v[b, h] = unit_kv(w, b, h)
    return k, v


def window_bits(w: Workload, k: np.ndarray) -> np.ndarray:
    """Bit width (8/4/2) per visual window, uint8 [W], from keys [1][Hkv][N][d]."""
    assert w.mixed and k.shape[0] == 1
    nv = w.windows * w.window_tokens
    keys = np.asarray(k[0], dtype=np.float64)                 # [Hkv][N][d]
    win = keys[:, :nv].reshape(w.n_kv_heads, w.windows, w.window_tokens, w.d_h)
    win_mean = win.mean(axis=2).transpose(1, 0, 2).reshape(w.windows, -1)   # [W][Hkv*d]
    txt_mean = keys[:, nv:nv + w.text_tokens].mean(axis=1).reshape(-1)      # [Hkv*d]
    cos = win_mean @ txt_mean / (np.linalg.norm(win_mean, axis=1) * np.linalg.norm(txt_mean))
    order = sorted(range(w.windows), key=lambda i: (-cos[i], i))
    n8 = int(np.floor(w.frac8 * w.windows))
    n84 = int(np.floor((w.frac8 + w.frac4) * w.windows))
    bits = np.full(w.windows, 2, dtype=np.uint8)
    for rank, i in enumerate(order):
        bits[i] = 8 if rank < n8 else (4 if rank < n84 else 2)
    return bits


def sample_units(w: Workload, n: int, seed: int = 1234):
    """``n`` distinct (b, h) streams, always including the first and last."""
    total = w.batch * w.n_kv_heads
    rng = np.random.default_rng([seed, 7])
    idx = {0, total - 1}
    if n > 2:
        idx.update(int(i) for i in rng.choice(total, size=min(n, total) - len(idx) + 2, replace=False))
    idx = sorted(idx)[:max(n, 2)]
    return [(i // w.n_kv_heads, i % w.n_kv_heads) for i in idx]


def search_tokens(batch: int, n_text: int, n_visual: int, dim: int, window_tokens: int,
                  seed: int = 0, prompt: float = 2.0, relevance_max: float = 3.0):
    """Synthetic encoder outputs for the window-level search, fp16.

    Stand-ins for the text-encoder tokens of a prompt and the vision-encoder
    tokens of a video (the pages use LLaVA-OneVision / Qwen2-VL features of
    real videos; none are available here).  A prompt direction u ~ N(0, I)
    (shared by the batch) is drawn from ``default_rng([seed, 5])``; text token
    = prompt * sqrt(D) * u/|u| + N(0, I); window i gets a relevance
    c_i ~ U(0, relevance_max) (shared by the batch) and each of its tokens is
    (c_i + N(0, 0.1)) * sqrt(D) * u/|u| + N(0, I), so the windows' scores
    spread over (0, 1) and the batch rows mostly agree.  Rows past the last
    full window get relevance 0.  Returns (text [B][N][D], visual [B][M][D]).
    """
    rng = np.random.default_rng([seed, 5])
    u = rng.standard_normal(dim)
    u = u / np.linalg.norm(u) * np.sqrt(dim)
    n_win = n_visual // window_tokens
    rel = np.zeros(n_visual)
    rel[:n_win * window_tokens] = np.repeat(rng.uniform(0, relevance_max, n_win), window_tokens)
    text = prompt * u + rng.standard_normal((batch, n_text, dim))
    jitter = rng.normal(0.0, 0.1, size=(batch, n_visual, 1))
    visual = (rel[None, :, None] + jitter) * u + rng.standard_normal((batch, n_visual, dim))
    return text.astype(np.float16), visual.astype(np.float16)


def ragged_contexts(n: int, lo: int = 512, hi: int = 8192, seed: int = 0) -> list:
    """Context lengths of a serving-shaped decode batch: ``n`` sequences whose
    cached lengths are log-uniform in [lo, hi] (``default_rng([seed, 6])``).
    The pages' serving runs (ShareGPT requests, long-document tasks) mix short
    and long sequences in one batch; this mix stands in for them."""
    rng = np.random.default_rng([seed, 6])
    x = np.exp(rng.uniform(np.log(lo), np.log(hi), size=n))
    return [int(v) for v in np.floor(x)]


def pq_inputs(batch: int, n_kv_heads: int, n_tok: int, d_h: int, m: int, bits: int, seed: int = 0):
    """PQ centroids and codes of a decode batch (PQCache note, "Method
    details", Step 2 shapes): centroids fp16 [B][Hkv][m][2^bits][d_h/m] drawn
    N(0, 1/m) (so a rebuilt key has about unit variance per channel), codes
    uint8 [B][Hkv][n_tok][m] uniform in [0, 2^bits); ``default_rng([seed, 8])``.
    K-means construction is not part of the path: these stand in for its
    output."""
    rng = np.random.default_rng([seed, 8])
    dm = d_h // m
    c = rng.standard_normal((batch, n_kv_heads, m, 1 << bits, dm), dtype=np.float32) / np.float32(np.sqrt(m))
    codes = rng.integers(0, 1 << bits, size=(batch, n_kv_heads, n_tok, m), dtype=np.uint8)
    return c.astype(np.float16), codes


def vq_inputs(batch: int, n_kv_heads: int, n_tok: int, d_h: int, rounds: int, seed: int = 0):
    """Codebooks and codes of a vector-quantized KV cache (VQ-LLM note, the
    CQ configurations: 4-channel sub-vectors, 256 entries each, ``rounds``
    residual rounds).  Codebooks fp16 [Hkv][rounds][d_h/4][256][4] for keys
    and for values, round r drawn N(0, 4^-r) (a residual round codes a
    smaller remainder); codes uint8 [B][Hkv][n_tok][rounds][d_h/4] uniform;
    ``default_rng([seed, 9])``.  Trained codebooks are not part of the path:
    these stand in for them."""
    rng = np.random.default_rng([seed, 9])
    G = d_h // 4
    scale = (0.5 ** np.arange(rounds, dtype=np.float32))[:, None, None, None]
    kb = rng.standard_normal((n_kv_heads, rounds, G, 256, 4), dtype=np.float32) * scale
    vb = rng.standard_normal((n_kv_heads, rounds, G, 256, 4), dtype=np.float32) * scale
    kc = rng.integers(0, 256, size=(batch, n_kv_heads, n_tok, rounds, G), dtype=np.uint8)
    vc = rng.integers(0, 256, size=(batch, n_kv_heads, n_tok, rounds, G), dtype=np.uint8)
    return kb.astype(np.float16), vb.astype(np.float16), kc, vc
