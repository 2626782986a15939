"""GPU parity of decode attention over a vector-quantized (codebook) KV cache
(kvq_vq_decode_attn) against the oracle (oracle/vq.py): every output within
2e-3 abs + 1e-3 rel of the float64 oracle (tests/helpers.py).  Shapes cover
both head dims, one and two rounds (CQ-2 / CQ-4), MHA and 2-16 query heads
per kv head, one chunk per stream (output written directly) and many
chunks (partial states and the merge kernel), ragged chunk tails, a single
token, and the Llama-2-7B decode shape at full size (sampled heads)."""
import numpy as np
import pytest

import workloads
from oracle import vq
from tests.helpers import assert_close, ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvq():
    ensure_built()
    import decode_attention_kivi_amd as m
    return m


def run_vq(kvq, B, Hq, Hkv, d, R, n, heads=None, seed=0):
    import torch
    dev = torch.device("cuda:0")
    print(f"vq: B{B} Hq{Hq} Hkv{Hkv} d{d} R{R} n{n}", flush=True)
    w = workloads.Workload(name="vq", batch=B, n_q_heads=Hq, n_kv_heads=Hkv, d_h=d, context=n,
                           group=32, residual=32, bits=2, seed=seed)
    q = workloads.queries(w)
    kb, vb, kc, vc = workloads.vq_inputs(B, Hkv, n, d, R, seed=seed)
    tb = R * d // 4
    stride = (n * tb + 15) // 16 * 16 + 16           # a stride past the codes
    def pad(c):
        x = np.full((B * Hkv, stride), 0xCD, np.uint8)
        x[:, :n * tb] = c.reshape(B * Hkv, n * tb)
        return torch.from_numpy(x).to(dev)
    ws_bytes = kvq.kvq_vq_decode_attn_workspace(B, Hq, Hkv, d, R, n)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=dev)
    scale = 1.0 / np.sqrt(d)
    kvq.kvq_vq_decode_attn(B, Hq, Hkv, d, R, n, scale, torch.from_numpy(q).to(dev), pad(kc), pad(vc), stride,
                           torch.from_numpy(kb).to(dev), torch.from_numpy(vb).to(dev), out,
                           ws if ws_bytes else None, ws_bytes)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    g = Hq // Hkv
    heads = heads or [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in heads:
        kv = h // g
        ref = vq.vq_attention(q[b, h:h + 1], kc[b, kv], vc[b, kv], kb[kv], vb[kv], scale)[0]
        assert_close(out[b, h], ref, f"vq ({b},{h})")
    return ws_bytes


@pytest.mark.parametrize("B,Hq,Hkv,d,R,n", [
    (1, 4, 4, 64, 1, 100),
    (2, 8, 2, 128, 2, 5000),
    (1, 28, 4, 128, 1, 3000),
    (3, 6, 2, 64, 2, 33),
    (1, 2, 1, 128, 2, 40000),
    (2, 4, 4, 128, 1, 1),
    (1, 8, 1, 64, 1, 4097),
    # many query heads per kv head (the kernel loops over them) and chunks
    (1, 16, 1, 128, 1, 9000),
    (2, 16, 2, 64, 2, 17000),
])
def test_vq_decode(kvq, B, Hq, Hkv, d, R, n):
    run_vq(kvq, B, Hq, Hkv, d, R, n)


def test_vq_decode_many_chunks_use_the_merge(kvq):
    # one stream of 20000 tokens: 79 chunks of 256 tokens, so the partial
    # states and the merge kernel are used
    assert run_vq(kvq, 1, 1, 1, 128, 1, 20000) > 0


def test_vq_decode_llama2_7b_full_size(kvq):
    # CQ-2 at the Llama-2-7B decode shape: 16 x 32 heads, 4097 tokens; one
    # chunk per stream (no partial states), sampled heads checked
    assert run_vq(kvq, 16, 32, 32, 128, 1, 4097,
                  heads=[(0, 0), (3, 17), (9, 31), (15, 5), (15, 30)]) == 0
