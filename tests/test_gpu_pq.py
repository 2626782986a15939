"""GPU parity of the PQCache decode-time PQ search (kvq_pq_search) against
the oracle (oracle/pq.py).

* scores within the fp32 error bound of their sums: |gpu - oracle| <=
  1e-5 * sum_j sum_d |q_jd c_jd| + 1e-6 per token (fp32 accumulation of at
  most 128 products and 16 table entries stays far inside it);
* the Top-k set is exact for the kernel's own scores: the oracle's Top-k
  rule (largest first, ties to the lower index, ascending order) applied to
  the returned fp32 scores gives the returned indices bit for bit;
* and valid for the oracle's scores: no token left out scores more than the
  tolerance above a chosen one.
Shapes cover 1-8 query heads per kv head (7 included), m = 1..16, 3..8-bit
codes, k = 1 and k = n_tok, token counts that are not multiples of the
16-byte code loads, both paths (a head's scores resident in LDS up to about
38K tokens, scores then Top-k through memory past that), and the GQA
long-context shape at full size (sampled heads checked); threshold ties
beyond the candidate list, and ties within it scattered over every wave's
token segment with the cut inside one.
"""
import numpy as np
import pytest

import workloads
from tests.helpers import ensure_built
from oracle import pq

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvq():
    ensure_built()
    import decode_attention_kivi_amd as m
    return m


def run_pq(kvq, B, Hq, Hkv, d, m, bits, n_tok, k, heads=None, seed=0, prepare=None):
    print(f"pq: B{B} Hq{Hq} Hkv{Hkv} d{d} m{m} bits{bits} n{n_tok} k{k}", flush=True)
    w = workloads.Workload(name="pq", batch=B, n_q_heads=Hq, n_kv_heads=Hkv, d_h=d, context=n_tok,
                           group=32, residual=32, bits=2, seed=seed)
    q = workloads.queries(w)
    c, codes = workloads.pq_inputs(B, Hkv, n_tok, d, m, bits, seed=seed)
    if prepare:
        prepare(q, c, codes)
    check_pq(kvq, q, c, codes, B, Hq, Hkv, d, m, bits, n_tok, k, heads)


def check_pq(kvq, q, c, codes, B, Hq, Hkv, d, m, bits, n_tok, k, heads=None):
    import torch
    dev = torch.device("cuda:0")
    stride = (n_tok * m + 15) // 16 * 16
    padded = np.full((B * Hkv, stride), 0xAB, np.uint8)          # padding bytes are read and ignored
    padded[:, :n_tok * m] = codes.reshape(B * Hkv, n_tok * m)
    qt = torch.from_numpy(q).to(dev)
    ct = torch.from_numpy(c).to(dev)
    kt = torch.from_numpy(padded).to(dev)
    sc = torch.empty(B, Hq, n_tok, dtype=torch.float32, device=dev)
    idx = torch.empty(B, Hq, k, dtype=torch.int32, device=dev)
    kvq.kvq_pq_search(B, Hq, Hkv, d, m, bits, n_tok, k, qt, ct, kt, stride, sc, idx)
    torch.cuda.synchronize()
    sc, idx = sc.cpu().numpy(), idx.cpu().numpy()
    g = Hq // Hkv
    heads = heads or [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in heads:
        kv = h // g
        cen = c[b, kv].astype(np.float64)
        ref = pq.pq_scores(q[b, h].astype(np.float64), cen, codes[b, kv])
        bound = pq.pq_scores(np.abs(q[b, h].astype(np.float64)), np.abs(cen), codes[b, kv])
        err = np.abs(sc[b, h].astype(np.float64) - ref) - (1e-5 * bound + 1e-6)
        assert np.all(err <= 0), f"scores ({b},{h}): max excess {err.max():.3e}"
        got = idx[b, h]
        assert got.tolist() == pq.topk_tokens(sc[b, h], k).tolist(), f"Top-k ({b},{h}) vs own scores"
        tol = float((1e-5 * bound + 1e-6).max())
        chosen = np.zeros(n_tok, bool)
        chosen[got] = True
        if chosen.all() or not chosen.any():
            continue
        assert ref[~chosen].max() <= ref[chosen].min() + 2 * tol, f"Top-k ({b},{h}) vs oracle scores"


@pytest.mark.parametrize("B,Hq,Hkv,d,m,bits,n_tok,k", [
    (1, 4, 4, 64, 2, 4, 100, 10),
    (2, 8, 2, 128, 2, 8, 5000, 500),
    (1, 4, 1, 128, 4, 6, 777, 777),
    (3, 6, 2, 128, 8, 3, 33, 1),
    (1, 28, 4, 128, 2, 8, 2049, 205),
    (2, 16, 2, 64, 1, 8, 300, 17),
    (1, 2, 1, 128, 16, 5, 4099, 64),
    # past the LDS-resident one-kernel path (about 38K tokens): scores
    # kernel, then the Top-k kernel through memory
    (1, 4, 2, 128, 2, 8, 40001, 999),
    (1, 2, 1, 64, 4, 4, 50000, 50000),
    # 1-bit codes, one sub-space: two score values, so thousands of tokens
    # tie at the threshold (more than the candidate list holds), both paths
    (1, 2, 1, 64, 1, 1, 20000, 5000),
    (1, 2, 1, 64, 1, 1, 60000, 7000),
    # more than 8 query heads per kv head: the fused path (one workgroup
    # per query head) and the scores kernel's head blocks of 8
    (1, 32, 1, 128, 2, 8, 3000, 300),
    (1, 32, 1, 128, 2, 8, 40001, 500),
    (2, 24, 2, 64, 4, 6, 40001, 100),
    # 8 heads x 16 sub-spaces of tables: the scores kernel's 512-thread form
    (1, 8, 1, 128, 16, 4, 40001, 300),
])
def test_pq_search(kvq, B, Hq, Hkv, d, m, bits, n_tok, k):
    run_pq(kvq, B, Hq, Hkv, d, m, bits, n_tok, k)


def test_pq_search_gqa_long_context_full_size(kvq):
    # the GQA long-context shape: 4 x 32 query heads over 8 kv heads, 32769
    # tokens, m = 2 sub-spaces of 256 centroids, Top-k = 1/10 of the tokens
    run_pq(kvq, 4, 32, 8, 128, 2, 8, 32769, 3277, heads=[(0, 0), (1, 13), (2, 31), (3, 7), (3, 24)])


def test_pq_search_ties(kvq):
    # every centroid of sub-space 0 equal and sub-space 1 two-valued: scores
    # take two values, so the threshold ties are broken by the token index
    import torch
    dev = torch.device("cuda:0")
    B, Hq, Hkv, d, m, bits, n, k = 1, 1, 1, 64, 2, 1, 50, 7
    q = np.ones((B, Hq, d), np.float16)
    c = np.zeros((B, Hkv, m, 2, d // m), np.float16)
    c[0, 0, 1, 1] = 1.0
    codes = np.zeros((B, Hkv, n, m), np.uint8)
    codes[0, 0, ::3, 1] = 1                                          # tokens 0, 3, 6, ... score 32
    stride = (n * m + 15) // 16 * 16
    padded = np.zeros((1, stride), np.uint8)
    padded[:, :n * m] = codes.reshape(1, -1)
    sc = torch.empty(B, Hq, n, dtype=torch.float32, device=dev)
    idx = torch.empty(B, Hq, k, dtype=torch.int32, device=dev)
    kvq.kvq_pq_search(B, Hq, Hkv, d, m, bits, n, k, torch.from_numpy(q).to(dev), torch.from_numpy(c).to(dev),
                      torch.from_numpy(padded).to(dev), stride, sc, idx)
    torch.cuda.synchronize()
    assert idx.cpu().numpy()[0, 0].tolist() == [0, 3, 6, 9, 12, 15, 18]
    k2 = 20                                                           # 17 at 32, then 3 of the zeros
    idx2 = torch.empty(B, Hq, k2, dtype=torch.int32, device=dev)
    kvq.kvq_pq_search(B, Hq, Hkv, d, m, bits, n, k2, torch.from_numpy(q).to(dev), torch.from_numpy(c).to(dev),
                      torch.from_numpy(padded).to(dev), stride, sc, idx2)
    torch.cuda.synchronize()
    assert idx2.cpu().numpy()[0, 0].tolist() == sorted(list(range(0, 50, 3)) + [1, 2, 4])


@pytest.mark.parametrize("n,n_ties", [(5000, 1000), (30000, 1400), (50000, 1000), (50001, 1400)])
def test_pq_search_ties_across_segments(kvq, n, n_ties):
    # scores 0, 64 and 96 only: 200 tokens at 96, n_ties tokens at 64 (fewer
    # than the candidate list holds) scattered over the whole range, so that
    # every wave's token segment holds some of them, and k takes all of the
    # 96s and the lower-index part of the 64s: the cut falls inside some
    # segment; both paths, 16-byte and 4-byte score reads on the memory path
    import torch
    dev = torch.device("cuda:0")
    B, Hq, Hkv, d, m, bits = 1, 1, 1, 64, 2, 1
    q = np.ones((B, Hq, d), np.float16)
    c = np.zeros((B, Hkv, m, 2, d // m), np.float16)
    c[0, 0, 0, 1] = 1.0                                              # sub-space 0, code 1: 32
    c[0, 0, 1, 1] = 2.0                                              # sub-space 1, code 1: 64
    perm = np.random.default_rng(n).permutation(n)
    top, ties = perm[:200], perm[200:200 + n_ties]
    codes = np.zeros((B, Hkv, n, m), np.uint8)
    codes[0, 0, top, :] = 1
    codes[0, 0, ties, 1] = 1
    k = 200 + n_ties // 2
    stride = (n * m + 15) // 16 * 16
    padded = np.zeros((1, stride), np.uint8)
    padded[:, :n * m] = codes.reshape(1, -1)
    sc = torch.empty(B, Hq, n, dtype=torch.float32, device=dev)
    idx = torch.empty(B, Hq, k, dtype=torch.int32, device=dev)
    print(f"pq ties across segments: n{n} ties{n_ties} k{k}", flush=True)
    kvq.kvq_pq_search(B, Hq, Hkv, d, m, bits, n, k, torch.from_numpy(q).to(dev), torch.from_numpy(c).to(dev),
                      torch.from_numpy(padded).to(dev), stride, sc, idx)
    torch.cuda.synchronize()
    want_sc = np.zeros(n, np.float32)
    want_sc[ties] = 64.0
    want_sc[top] = 96.0
    assert np.array_equal(sc.cpu().numpy()[0, 0], want_sc)
    want = sorted(top.tolist() + sorted(ties.tolist())[:n_ties // 2])
    assert idx.cpu().numpy()[0, 0].tolist() == want


def test_pq_search_outlier_score(kvq):
    # one token far above the rest stretches the score range, so the others
    # crowd into one or two of the 2048 equal-width level-1 buckets and the
    # threshold is found through the level-2 buckets
    def prepare(q, c, codes):
        g, dm = q.shape[1] // c.shape[1], c.shape[-1]
        c[:, :, 0, 0, :] = np.float16(1000.0) * np.sign(q[:, ::g, :dm].astype(np.float32)).astype(np.float16)
        codes[:, :, :, 0] = np.maximum(codes[:, :, :, 0], 1)         # centroid 0 of sub-space 0 ...
        codes[:, :, 777, 0] = 0                                       # ... for token 777 only
    run_pq(kvq, 1, 4, 2, 64, 1, 8, 30000, 2500, prepare=prepare)
    run_pq(kvq, 1, 2, 1, 128, 2, 8, 45000, 3000, prepare=prepare)
