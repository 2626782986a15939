"""Shared helpers of the tests (no test functions here)."""
import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "decode_attention_kivi_amd", "libkvq.so")

# attention tolerance: 2e-3 max-abs plus 1e-3 relative, element by element
ATOL, RTOL = 2e-3, 1e-3


def ensure_built():
    if not os.path.exists(LIB):
        from decode_attention_kivi_amd import build
        build.build()


def assert_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    excess = np.abs(got - ref) - (ATOL + RTOL * np.abs(ref))
    if np.any(excess > 0):
        i = np.unravel_index(np.argmax(excess), excess.shape)
        raise AssertionError(f"{what}: |gpu-oracle| = {abs(got[i] - ref[i]):.3e} at {i} "
                             f"(gpu {got[i]:.6f}, oracle {ref[i]:.6f}); tol {ATOL}+{RTOL}*|ref|")
    return float(np.max(np.abs(got - ref))) if got.size else 0.0
