"""kvq_decode_attn_noalloc (partial states in the library's static device
scratch) against kvq_decode_attn (partial states in a caller workspace):
the same kernels, so the outputs must be bit-identical.  Two calls in a row
on one GPU, the second on a smaller cache with fewer partial states, so
stale scratch contents from the first call would show.  Both shapes need
several workgroups per stream (a non-empty workspace), or the scratch
would go unused."""
import numpy as np
import pytest
import torch

from tests.helpers import assert_close, ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvq():
    ensure_built()
    import decode_attention_kivi_amd as m
    return m


def build_cache(B, Hkv, d, L, bits, G, R, seed):
    from decode_attention_kivi_amd.cache import KiviCache
    dev = torch.device("cuda")
    g = torch.Generator(device=dev).manual_seed(seed)
    k = torch.randn(B, Hkv, L + 1, d, generator=g, device=dev).half()
    v = torch.randn(B, Hkv, L + 1, d, generator=g, device=dev).half()
    c = KiviCache(B, Hkv, d, bits, G, R, L + 1, dev)
    c.prefill(k[:, :, :L], v[:, :, :L])
    c.append(k[:, :, L:L + 1], v[:, :, L:L + 1])
    return c


@pytest.mark.parametrize("case", [
    # (B, Hq, Hkv, d, L, bits, G, R) for the first and the second call
    ((2, 8, 2, 128, 24000, 2, 64, 128), (1, 4, 1, 128, 9000, 2, 64, 128)),
    ((1, 28, 4, 128, 20000, 4, 32, 128), (1, 8, 2, 64, 5000, 8, 32, 64)),
])
def test_noalloc_matches_workspace_call(kvq, case):
    for i, (B, Hq, Hkv, d, L, bits, G, R) in enumerate(case):
        print(f"noalloc call {i}: B{B} Hq{Hq} Hkv{Hkv} d{d} L{L} int{bits} G{G} R{R}", flush=True)
        c = build_cache(B, Hkv, d, L, bits, G, R, seed=10 + i)
        q = torch.randn(B, Hq, d, generator=torch.Generator(device="cuda").manual_seed(20 + i),
                        device="cuda").half()
        sm = 1.0 / d ** 0.5
        ref = torch.empty(B, Hq, d, dtype=torch.float32, device="cuda")
        got = torch.full_like(ref, float("nan"))
        a = c.decode_args(q, ref, sm)
        need = kvq.kvq_decode_attn_workspace(a)
        assert 0 < need <= kvq.KVQ_SCRATCH_BYTES, need
        kvq.kvq_decode_attn(a)
        a.out = got.data_ptr()
        a.workspace = None                      # ignored by the no-alloc call
        a.workspace_bytes = 0
        kvq.kvq_decode_attn_noalloc(a)
        torch.cuda.synchronize()
        r, o = ref.cpu().numpy(), got.cpu().numpy()
        assert np.all(np.isfinite(o))
        assert_close(o, r, "noalloc vs workspace call")
        assert np.array_equal(o.view(np.uint32), r.view(np.uint32)), "not bit-identical"
