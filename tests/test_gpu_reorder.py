"""GPU parity of kvq_reorder_windows against the oracle: permutation, run
table and gather list bit-exact (WindowQuant Sec. 3.3.1)."""
import numpy as np
import pytest

from tests.helpers import ensure_built
from oracle import windows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvq():
    ensure_built()
    import decode_attention_kivi_amd as m
    return m


def _reorder(kvq, bits, S, G, d, gather=True):
    import torch
    dev = torch.device("cuda")
    W = len(bits)
    wb = torch.tensor(np.asarray(bits, np.uint8), device=dev)
    perm = torch.full((W,), -1, dtype=torch.int32, device=dev)
    segs = torch.zeros(128, dtype=torch.uint8, device=dev)
    ns = torch.zeros(1, dtype=torch.int32, device=dev)
    rg = torch.full((W * S,), -1, dtype=torch.int32, device=dev) if gather else None
    print(f"reorder W={W} S={S} G={G} d={d}", flush=True)
    kvq.kvq_reorder_windows(wb, W, S, G, d, perm, segs, ns, rg)
    torch.cuda.synchronize()
    n = int(ns.cpu().item())
    raw = segs.cpu().numpy().tobytes()
    seg_rows = [kvq.Segment.from_buffer_copy(raw[32 * i:32 * i + 32]).astuple() for i in range(max(n, 0))]
    return n, perm.cpu().numpy(), seg_rows, (rg.cpu().numpy() if gather else None)


@pytest.mark.parametrize("W", [1, 5, 128, 1000, 3000])
@pytest.mark.parametrize("S,G,d", [(256, 32, 128), (64, 64, 64), (128, 128, 128)])
def test_reorder_bit_exact(kvq, W, S, G, d):
    rng = np.random.default_rng([W, S])
    bits = rng.choice([16, 8, 4, 2], size=W, p=[0.05, 0.1, 0.3, 0.55]).astype(np.uint8)
    n, perm, segs, rg = _reorder(kvq, bits, S, G, d, gather=W * S <= 1 << 20)
    assert perm.tolist() == windows.reorder(bits)
    assert n == len(windows.segment_table(bits, S, d, G))
    assert [tuple(s) for s in segs] == [tuple(s) for s in windows.segment_table(bits, S, d, G)]
    if rg is not None:
        assert np.array_equal(rg, windows.row_gather(windows.reorder(bits), S))


def test_reorder_max_windows_one_width(kvq):
    bits = np.full(65536, 4, np.uint8)
    bits[::7] = 2
    n, perm, segs, _ = _reorder(kvq, bits, 32, 32, 64, gather=False)
    assert perm.tolist() == windows.reorder(bits)
    assert [tuple(s) for s in segs] == [tuple(s) for s in windows.segment_table(bits, 32, 64, 32)]


def test_reorder_rejects_bad_width_on_device(kvq):
    bits = np.array([2, 4, 3, 8], np.uint8)
    n, _, _, _ = _reorder(kvq, bits, 64, 32, 128)
    assert n == -1


def test_two_runs_bit_identical(kvq):
    """Determinism: the same widths give the same permutation, run table and
    gather list, run after run (the gather list comes from a grid-wide
    kernel over W * S entries)."""
    rng = np.random.default_rng(11)
    bits = rng.choice([16, 8, 4, 2], size=3000, p=[0.05, 0.1, 0.3, 0.55]).astype(np.uint8)
    a = _reorder(kvq, bits, 256, 32, 128)
    b = _reorder(kvq, bits, 256, 32, 128)
    assert a[0] == b[0] and a[2] == b[2]
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[3], b[3])
