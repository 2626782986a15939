"""GPU parity of decode attention over a paged, ragged KIVI cache
(kvq_decode_attn_paged) against the oracle, sequence by sequence.

Each sequence of the batch has its own context length; its state is a KIVI
prefill of that many tokens followed by one decode step.  The quantized
tokens live in pages taken from a shuffled pool (the block table is a real
indirection).  The oracle runs the same prefill + decode step per (sequence,
kv head) stream and its float64 attention is the expected output: within
2e-3 abs + 1e-3 rel.  Lengths cover the empty and sub-R prefill, page and
group boundaries, odd value counts, and sequences long enough to need
several workgroups (partial states merged by the second kernel).
"""
import numpy as np
import pytest

import workloads
from tests.helpers import assert_close, ensure_built
from oracle.kivi import KiviStream

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvq():
    ensure_built()
    import decode_attention_kivi_amd as m
    return m


def run_paged(contexts, n_q_heads, n_kv_heads, d, G, R, bits, page_tokens, n_out=0, factor=1.0, seed=0):
    import torch
    from decode_attention_kivi_amd.cache import PagedKiviCache, kivi_step_lengths
    dev = torch.device("cuda:0")
    B = len(contexts)
    w = workloads.Workload(name="paged", batch=B, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, d_h=d,
                           context=max(contexts), group=G, residual=R, bits=bits, n_outlier=n_out,
                           outlier_factor=factor, seed=seed)
    print(f"paged: B{B} Hq{n_q_heads} Hkv{n_kv_heads} d{d} G{G} R{R} b{bits} PT{page_tokens} "
          f"contexts={list(contexts)}", flush=True)
    cache = PagedKiviCache(B, n_kv_heads, d, bits, G, R, page_tokens, max(contexts) + 1, device=dev,
                           seed=seed + 1)
    kv = {}
    for b, L in enumerate(contexts):
        pairs = [workloads.unit_kv(w, b, h, n_tokens=L + 1) for h in range(n_kv_heads)]
        k = np.stack([p[0] for p in pairs])
        v = np.stack([p[1] for p in pairs])
        kv[b] = (k, v)
        cache.fill_step(b, torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev))
    q = workloads.queries(w)
    out = cache.attend(torch.from_numpy(q).to(dev), w.sm_scale).cpu().numpy()
    torch.cuda.synchronize()
    g = n_q_heads // n_kv_heads
    worst = 0.0
    for b, L in enumerate(contexts):
        k, v = kv[b]
        n_kq, r_k, n_vq, r_v = kivi_step_lengths(L, R)
        assert tuple(cache.lens[b]) == (n_kq, n_vq, r_k, r_v)
        for h in range(n_kv_heads):
            st = KiviStream(d, bits, G, R)
            st.prefill(k[h, :L], v[h, :L])
            st.decode_append(k[h, L], v[h, L])
            assert st.lengths == (n_kq, r_k, n_vq, r_v), (st.lengths, (n_kq, r_k, n_vq, r_v))
            ref = st.attend(q[b, h * g:(h + 1) * g], w.sm_scale)
            worst = max(worst, assert_close(out[b, h * g:(h + 1) * g], ref, f"seq {b} (L={L}) head {h}"))
    return worst


def test_ragged_mha_int2(kvq):
    # R = 32 keeps the oracle cheap; lengths straddle pages (256) and groups
    run_paged([0, 1, 31, 32, 63, 255, 256, 257, 700, 1023], 4, 4, 128, 32, 32, 2, 256,
              n_out=3, factor=8.0)


def test_ragged_long_sequences_merge(kvq):
    # one sequence long enough for several workgroups: every stream goes
    # through the partial-state workspace and the merge kernel
    run_paged([9000, 130, 4500], 2, 2, 128, 32, 128, 2, 512, n_out=3, factor=8.0)


@pytest.mark.parametrize("bits", [4, 8])
def test_ragged_gqa_wider_codes(kvq, bits):
    run_paged([5, 200, 640, 1500], 8, 2, 128, 64, 128, bits, 128)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 1), (6, 2)])
def test_ragged_d64(kvq, hq, hkv):
    run_paged([3, 100, 333, 1200], hq, hkv, 64, 32, 32, 2, 64)


@pytest.mark.parametrize("hq,hkv,d", [(32, 1, 128), (24, 2, 64)])
def test_ragged_many_query_heads(kvq, hq, hkv, d):
    # more than 4 query heads per kv head: head blocks of 4
    run_paged([5, 300, 2000], hq, hkv, d, 32, 32, 2, 256, n_out=3, factor=8.0)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("hq,hkv", [(2, 2), (8, 2)])
def test_wave_ranges_across_many_pages(kvq, bits, hq, hkv):
    # 64-token pages at d_h 128: a wave's range crosses several pages, which
    # one load pipeline walks (page cursor); odd value counts end mid-pair
    run_paged([3, 701, 1500, 2900], hq, hkv, 128, 32, 64, bits, 64, n_out=3, factor=8.0)


def test_page_equals_group(kvq):
    # pages of 128 tokens with groups of 128 tokens: one key group per page
    run_paged([129, 384, 1000], 2, 2, 128, 128, 128, 4, 128)


def test_more_sequences_than_the_schedule(kvq):
    # above 256 sequences the grid is (workgroups per stream, streams) with
    # surplus workgroups leaving at once, instead of the sorted 1-D schedule
    rng = np.random.default_rng(3)
    run_paged([int(x) for x in rng.integers(0, 300, size=260)], 1, 1, 64, 32, 32, 2, 64)


def _random_case(seed: int):
    # page sizes are multiples of 64 and of G; G <= d; R a multiple of G
    rng = np.random.default_rng([seed, 78])
    d = int(rng.choice([64, 128]))
    G = int(rng.choice([32, 64] if d == 64 else [32, 64, 128]))
    R = G * int(rng.integers(1, 3))
    pt = int(np.lcm(64, G) * rng.integers(1, 5))
    hkv = int(rng.integers(1, 4))
    hq = hkv * int(rng.choice([1, 2, 3, 4, 7, 8]))
    n = int(rng.integers(1, 9))
    contexts = [int(x) for x in rng.integers(0, 3000, size=n)]
    if rng.integers(0, 2):
        contexts[0] = int(rng.integers(5000, 12000))      # a sequence that needs several workgroups
    return contexts, hq, hkv, d, G, R, int(rng.choice([2, 4, 8])), pt


@pytest.mark.parametrize("seed", range(8))
def test_random_paged_batches(kvq, seed):
    # seeded random batches: lengths, heads, GQA ratio, head dim, group,
    # residual, width and page size drawn together
    contexts, hq, hkv, d, G, R, bits, pt = _random_case(seed)
    run_paged(contexts, hq, hkv, d, G, R, bits, pt, n_out=2, factor=8.0, seed=seed)
