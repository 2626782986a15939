"""Seeded random shapes for the KIVI decode path against the oracle: batch,
kv heads, query heads per kv head (1-8, including ones that are not powers of
two), head dim, group size, residual length, bit width, context length
(including 0 and lengths that are not multiples of anything), several decode
steps, forced split sizes and the one-call step, drawn together so that
combinations the hand-picked cases do not cover are exercised; and random
mixed-width window caches (window count and size, group, head dim, GQA
ratio, trailing fp16 tokens, a width of 2/4/8/16 bits per window, forced
splits).  Cache bytes bit for bit and attention within 2e-3 abs + 1e-3 rel,
as in test_gpu_decode."""
import numpy as np
import pytest

import workloads
from tests.test_gpu_decode import kvq, run_kivi  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu


def _case(seed: int):
    rng = np.random.default_rng([seed, 77])
    d = int(rng.choice([64, 128]))
    G = int(rng.choice([32, 64]))
    R = G * int(rng.integers(1, 3))
    w = workloads.get("tiny").scaled(
        name=f"random{seed}", batch=int(rng.integers(1, 4)), n_kv_heads=int(rng.integers(1, 4)), d_h=d,
        group=G, residual=R, bits=int(rng.choice([2, 4, 8])), context=int(rng.integers(0, 900)),
        n_outlier=int(rng.integers(0, 4)), outlier_factor=float(rng.choice([1.0, 8.0])), seed=seed)
    w = w.scaled(n_q_heads=w.n_kv_heads * int(rng.choice([1, 2, 3, 4, 5, 7, 8])))
    steps = int(rng.choice([1, 2, 5]))
    one_call = bool(rng.integers(0, 2))
    split = 0 if one_call or rng.integers(0, 2) == 0 else int(rng.integers(64, 400))
    return w, steps, one_call, split


@pytest.mark.parametrize("seed", range(16))
def test_random_shapes(kvq, seed):  # noqa: F811
    w, steps, one_call, split = _case(seed)
    units = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    run_kivi(kvq, w, units, steps=steps, split_tokens=split, check_every_step=True, one_call=one_call)


def _window_case(seed: int):
    rng = np.random.default_rng([seed, 79])
    d = int(rng.choice([64, 128]))
    G = int(rng.choice([32, 64]))
    S = int(rng.choice([64, 128, 256]))
    W = int(rng.integers(2, 21))
    text = int(rng.integers(0, 71))
    hkv = int(rng.integers(1, 4))
    w = workloads.get("qwen2_7b_windows").scaled(
        name=f"windows{seed}", batch=int(rng.integers(1, 3)), n_kv_heads=hkv,
        n_q_heads=hkv * int(rng.choice([1, 2, 4, 7])), d_h=d, group=G, windows=W, window_tokens=S,
        text_tokens=text, context=W * S + text - 1, seed=seed)
    bits = [int(x) for x in rng.choice([2, 4, 8, 16], size=W, p=[0.4, 0.3, 0.2, 0.1])]
    split = 0 if rng.integers(0, 2) == 0 else int(rng.integers(64, 500))
    return w, bits, split


@pytest.mark.parametrize("seed", range(8))
def test_random_windows(kvq, seed):  # noqa: F811
    from tests.test_gpu_decode import run_windows
    w, bits, split = _window_case(seed)
    run_windows(kvq, w, bits, units=[(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)],
                split_tokens=split)
