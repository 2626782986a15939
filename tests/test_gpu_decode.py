"""GPU parity of the whole decode path (quantize-append, residual
bookkeeping, reorder, decode attention) against the oracle.

* every cache byte of the sampled streams is compared bit for bit (codes,
  scales, zero points, residual rows);
* attention within 2e-3 abs + 1e-3 rel of the float64 oracle;
* small shapes cover ragged lengths, several decode steps (key flushes and
  value-window compaction), forced split sizes, GQA ratios 1..8, head dims
  64/128 and mixed-width runs including an fp16 run;
* the five workloads run at their full sizes in the launch configuration the
  benchmark uses (automatic split size), the oracle checking sampled streams.
"""
import functools

import numpy as np
import pytest

import workloads
from tests.helpers import assert_close, ensure_built
from oracle import pack, windows
from oracle.kivi import KiviStream

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvq():
    ensure_built()
    import decode_attention_kivi_amd as m
    return m


def _kv(w: workloads.Workload, extra: int = 0):
    """Host fp16 keys/values [B][Hkv][N+extra][d] of a workload (cached by shape)."""
    return _kv_cached(w.scaled(name="", bits=0, n_q_heads=w.n_kv_heads, note=""), w.n_tokens + extra)


@functools.lru_cache(maxsize=2)
def _kv_cached(w: workloads.Workload, n: int):
    shape = (w.batch, w.n_kv_heads, n, w.d_h)
    k = np.empty(shape, np.float16)
    v = np.empty(shape, np.float16)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            k[b, h], v[b, h] = workloads.unit_kv(w, b, h, n_tokens=n)
    return k, v


def _check_stream_bytes(cache, s, st, w):
    d, bits, G = w.d_h, w.bits, w.group
    assert cache.lengths == st.lengths, (cache.lengths, st.lengths)
    n_kq, r_k, n_vq, r_v = st.lengths
    kc = cache.k_codes[s].cpu().numpy()
    km = cache.k_meta[s].cpu().numpy()
    vc = cache.v_codes[s].cpu().numpy()
    vm = cache.v_meta[s].cpu().numpy()
    e = pack.pack_rows(st.kq, bits).reshape(-1)
    assert np.array_equal(kc[:e.size], e), "key codes"
    e = pack.pack_key_meta(st.ks, st.kz).view(np.uint8)
    assert np.array_equal(km[:e.size], e), "key scale/zero"
    e = pack.pack_values(st.vq, bits).reshape(-1)
    assert np.array_equal(vc[:e.size], e), "value codes"
    e = pack.pack_value_meta(st.vs, st.vz).view(np.uint8)
    assert np.array_equal(vm[:e.size], e), "value scale/zero"
    kr = cache.k_res[s, :r_k].cpu().numpy()
    vr = cache.v_res[s, cache.v_start:cache.v_start + r_v].cpu().numpy()
    assert np.array_equal(kr.view(np.uint16), st.k_res.view(np.uint16)), "key residual"
    assert np.array_equal(vr.view(np.uint16), st.v_res.view(np.uint16)), "value residual"


def run_kivi(kvq, w, units, steps=1, split_tokens=0, check_every_step=False, bytes_units=None,
             one_call=False, launches=None):
    """Prefill w.context tokens, then `steps` decode steps; compare with the oracle.
    one_call: every step is one kvq_kivi_step (append, flushes and attention);
    `launches` (a list) then collects the kernel launches of every step."""
    import torch
    from decode_attention_kivi_amd.cache import KiviCache
    dev = torch.device("cuda")
    k, v = _kv(w, steps - 1)
    L = w.context
    q = workloads.queries(w)
    kt = torch.from_numpy(k).to(dev)
    vt = torch.from_numpy(v).to(dev)
    qt = torch.from_numpy(q).to(dev)
    print(f"kivi {w.name}: B{w.batch} Hq{w.n_q_heads} Hkv{w.n_kv_heads} d{w.d_h} L{L} G{w.group} "
          f"R{w.residual} b{w.bits} steps={steps} split={split_tokens}", flush=True)
    cache = KiviCache(w.batch, w.n_kv_heads, w.d_h, w.bits, w.group, w.residual, L + steps, dev)
    cache.prefill(kt[:, :, :L], vt[:, :, :L])
    streams = {u: KiviStream(w.d_h, w.bits, w.group, w.residual) for u in units}
    for (b, h), st in streams.items():
        st.prefill(k[b, h, :L], v[b, h, :L])
    g = w.gqa
    worst = 0.0
    for step in range(steps):
        t = L + step
        if one_call:
            out = cache.step(kt[:, :, t:t + 1], vt[:, :, t:t + 1], qt, w.sm_scale)
            if launches is not None:
                launches.append(cache.last_launches)
        else:
            cache.append(kt[:, :, t:t + 1], vt[:, :, t:t + 1])
        for (b, h), st in streams.items():
            st.decode_append(k[b, h, t], v[b, h, t])
        if not (check_every_step or step == steps - 1):
            continue
        if not one_call:
            out = cache.attend(qt, w.sm_scale, split_tokens=split_tokens)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        assert np.all(np.isfinite(o))
        for (b, h), st in streams.items():
            if bytes_units is None or (b, h) in bytes_units:
                _check_stream_bytes(cache, b * w.n_kv_heads + h, st, w)
            ref = st.attend(q[b, h * g:(h + 1) * g], w.sm_scale)
            worst = max(worst, assert_close(o[b, h * g:(h + 1) * g], ref, f"{w.name} step {step} b{b} h{h}"))
    return worst


# -- small shapes: edge cases ------------------------------------------------------
SMALL = workloads.get("tiny")


@pytest.mark.parametrize("L", [0, 1, 5, 31, 32, 63, 100, 255, 256, 257])
def test_ragged_lengths(kvq, L):
    w = SMALL.scaled(context=L, batch=2)
    run_kivi(kvq, w, units=[(b, h) for b in range(2) for h in range(4)])


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_many_steps_flush_and_window(kvq, bits):
    w = SMALL.scaled(context=40, bits=bits, residual=32, n_kv_heads=2, n_q_heads=2)
    run_kivi(kvq, w, units=[(0, 0), (0, 1)], steps=3 * 32 + 5, check_every_step=True)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_one_call_steps(kvq, bits):
    # kvq_kivi_step: append, value-window overflow, key flush every R steps,
    # window compaction and attention in one call, checked after every step
    w = SMALL.scaled(context=40, bits=bits, residual=32, n_kv_heads=2, n_q_heads=4)
    launches = []
    run_kivi(kvq, w, units=[(0, 0), (0, 1)], steps=3 * 32 + 5, check_every_step=True, one_call=True,
             launches=launches)
    assert max(launches) >= 3          # flush steps: append, flush, attention


@pytest.mark.parametrize("context", [0, 1, 127, 128])
def test_one_call_steps_d128_gqa(kvq, context):
    w = SMALL.scaled(context=context, d_h=128, group=32, residual=128, n_kv_heads=2, n_q_heads=16,
                     batch=2)
    launches = []
    run_kivi(kvq, w, units=[(1, 0), (1, 1)], steps=140, check_every_step=True, one_call=True,
             launches=launches)
    assert max(launches) >= 3                        # flush steps
    if context < 64:
        # until the value window overflows, the tokens an append writes lie in
        # the last wave's range: those steps run fused
        assert 1 in launches


@pytest.mark.parametrize("bits,d", [(2, 128), (4, 128), (8, 128), (2, 64)])
def test_one_call_fused_steps_long_context(kvq, bits, d):
    # the value window overflows every step and the last wave's range holds
    # the residual and the value being quantized: the fused launch quantizes
    # the oldest window value and attends in one kernel
    w = SMALL.scaled(context=3 * 256 + 100, d_h=d, bits=bits, group=32, residual=32, n_kv_heads=2,
                     n_q_heads=4, batch=1)
    launches = []
    run_kivi(kvq, w, units=[(0, 0), (0, 1)], steps=40, check_every_step=True, one_call=True,
             launches=launches)
    assert launches.count(1) >= 30, launches


def test_one_call_steps_many_streams(kvq):
    # 20 x 32 streams, more than two 8-wave workgroups per CU hold: the plan
    # takes 4-wave workgroups, and the fused step's append runs in the last
    # of the 4 waves; checked after every step through a key flush
    w = SMALL.scaled(context=100, d_h=128, group=32, residual=32, n_kv_heads=32, n_q_heads=32,
                     batch=20)
    launches = []
    run_kivi(kvq, w, units=[(0, 0), (7, 31), (19, 5)], steps=40, check_every_step=True, one_call=True,
             launches=launches)
    assert 1 in launches and max(launches) >= 3


@pytest.mark.parametrize("split", [2, 33, 64, 96, 1000])
def test_forced_split_sizes(kvq, split):
    w = SMALL.scaled(context=700, n_kv_heads=2, n_q_heads=2)
    run_kivi(kvq, w, units=[(0, 0), (0, 1)], split_tokens=split)


def test_workspace_reused_across_splits(kvq):
    """One cache (one workspace) serves calls whose split changes (64, 128,
    automatic, 96, 64 tokens per workgroup, each merged across its
    workgroups) and then calls with another query-head count: every result
    matches the oracle."""
    import torch
    from decode_attention_kivi_amd.cache import KiviCache
    dev = torch.device("cuda")
    w = SMALL.scaled(context=700, n_kv_heads=2, n_q_heads=4)
    k, v = _kv(w)
    L = w.context
    cache = KiviCache(w.batch, w.n_kv_heads, w.d_h, w.bits, w.group, w.residual, L + 1, dev)
    cache.prefill(torch.from_numpy(k[:, :, :L]).to(dev), torch.from_numpy(v[:, :, :L]).to(dev))
    streams = {}
    for h in range(w.n_kv_heads):
        st = KiviStream(w.d_h, w.bits, w.group, w.residual)
        st.prefill(k[0, h, :L], v[0, h, :L])
        streams[h] = st
    for hq, splits in [(4, [64, 128, 0, 96, 64]), (8, [64, 96])]:
        wq = w.scaled(n_q_heads=hq)
        q = workloads.queries(wq)
        g = hq // w.n_kv_heads
        for split in splits:
            print(f"workspace reuse: Hq{hq} split={split}", flush=True)
            out = cache.attend(torch.from_numpy(q).to(dev), w.sm_scale, split_tokens=split)
            torch.cuda.synchronize()
            o = out.cpu().numpy()
            for h, st in streams.items():
                assert_close(o[0, h * g:(h + 1) * g], st.attend(q[0, h * g:(h + 1) * g], w.sm_scale),
                             f"Hq{hq} split {split} h{h}")


@pytest.mark.parametrize("hq,hkv", [(2, 1), (4, 1), (8, 2), (7, 1), (6, 2), (16, 2)])
@pytest.mark.parametrize("d,G", [(64, 32), (128, 64)])
def test_gqa_and_head_dims(kvq, hq, hkv, d, G):
    w = SMALL.scaled(n_q_heads=hq, n_kv_heads=hkv, d_h=d, group=G, residual=2 * G, context=5 * G + 7)
    run_kivi(kvq, w, units=[(0, h) for h in range(hkv)])


@pytest.mark.parametrize("bits", [4, 8])
def test_head_dim_128_wider_codes(kvq, bits):
    w = SMALL.scaled(d_h=128, bits=bits, group=32, residual=64, context=333)
    run_kivi(kvq, w, units=[(0, h) for h in range(4)])


# -- mixed-width runs (WindowQuant) --------------------------------------------------
def run_windows(kvq, w, bits_list, units, split_tokens=0, check_bytes=True):
    import torch
    from decode_attention_kivi_amd.cache import WindowCache
    dev = torch.device("cuda")
    k, v = _kv(w)
    q = workloads.queries(w)
    win_bits = np.asarray(bits_list, np.uint8)
    print(f"windows {w.name}: W{len(win_bits)} S{w.window_tokens} Hq{w.n_q_heads} Hkv{w.n_kv_heads} "
          f"G{w.group} split={split_tokens}", flush=True)
    kt = torch.from_numpy(k).to(dev)
    vt = torch.from_numpy(v).to(dev)
    cache = WindowCache(kt, vt, torch.from_numpy(win_bits).to(dev), w.window_tokens, w.group)
    out = cache.attend(torch.from_numpy(q).to(dev), w.sm_scale, split_tokens=split_tokens)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(np.isfinite(o))
    perm = windows.reorder(win_bits)
    assert cache.perm.cpu().numpy().tolist() == perm
    segs = windows.segment_table(win_bits, w.window_tokens, w.d_h, w.group)
    assert [tuple(s) for s in cache.segs] == [tuple(s) for s in segs]
    g = w.gqa
    worst = 0.0
    for (b, h) in units:
        st = windows.WindowStream(k[b, h], v[b, h], win_bits, w.window_tokens, w.group)
        s = b * w.n_kv_heads + h
        if check_bytes:
            kc, km = cache.k_codes[s].cpu().numpy(), cache.k_meta[s].cpu().numpy()
            vc, vm = cache.v_codes[s].cpu().numpy(), cache.v_meta[s].cpu().numpy()
            for seg, (bits, kp, vp) in zip(segs, st.runs):
                if bits == 16:
                    e = kp.view(np.uint8).reshape(-1)
                    assert np.array_equal(kc[seg.code_off:seg.code_off + e.size], e)
                    e = vp.view(np.uint8).reshape(-1)
                    assert np.array_equal(vc[seg.code_off:seg.code_off + e.size], e)
                    continue
                e = pack.pack_rows(kp[0], bits).reshape(-1)
                assert np.array_equal(kc[seg.code_off:seg.code_off + e.size], e), f"key codes {bits}"
                e = pack.pack_key_meta(kp[1], kp[2]).view(np.uint8)
                assert np.array_equal(km[seg.meta_off:seg.meta_off + e.size], e), f"key meta {bits}"
                e = pack.pack_values(vp[0], bits).reshape(-1)
                assert np.array_equal(vc[seg.code_off:seg.code_off + e.size], e), f"value codes {bits}"
                e = pack.pack_value_meta(vp[1], vp[2]).view(np.uint8)
                assert np.array_equal(vm[seg.meta_off:seg.meta_off + e.size], e), f"value meta {bits}"
        ref = st.attend(q[b, h * g:(h + 1) * g], w.sm_scale)
        worst = max(worst, assert_close(o[b, h * g:(h + 1) * g], ref, f"{w.name} b{b} h{h}"))
    return worst


@pytest.mark.parametrize("split", [0, 64, 100])
def test_mixed_windows_small(kvq, split):
    w = workloads.get("qwen2_7b_windows").scaled(windows=9, window_tokens=64, text_tokens=11,
                                                 context=9 * 64 + 11, n_q_heads=8, n_kv_heads=2, batch=2)
    bits = [2, 8, 16, 4, 2, 2, 8, 4, 16]
    run_windows(kvq, w, bits, units=[(b, h) for b in range(2) for h in range(2)], split_tokens=split)


def test_windows_no_residual_d64(kvq):
    w = workloads.get("qwen2_7b_windows").scaled(windows=6, window_tokens=64, text_tokens=0,
                                                 context=6 * 64 - 1, n_q_heads=4, n_kv_heads=4, d_h=64)
    # N = W*S exactly: context = W*S - 1 so that the decode token is the last window token
    run_windows(kvq, w, [4, 2, 8, 2, 4, 8], units=[(0, h) for h in range(4)])


# -- the five workloads at full size ---------------------------------------------------
def test_workload_tiny_full(kvq):
    w = workloads.get("tiny")
    run_kivi(kvq, w, units=[(0, h) for h in range(w.n_kv_heads)])


@pytest.mark.parametrize("name", ["llama2_7b", "llama2_7b_b64_int2", "llama2_7b_b64_int4",
                                  "llama31_8b_gqa"])
def test_workload_full_size_sampled(kvq, name):
    w = workloads.get(name)
    units = workloads.sample_units(w, 6)
    worst = run_kivi(kvq, w, units=units, bytes_units=set(units[:3]))
    print(f"{name}: max |gpu - oracle| = {worst:.3e}", flush=True)


def test_workload_windows_full(kvq):
    w = workloads.get("qwen2_7b_windows")
    k, _ = _kv(w)
    bits = workloads.window_bits(w, k)
    assert sorted(bits.tolist()).count(8) == 12 and sorted(bits.tolist()).count(4) == 39
    run_windows(kvq, w, bits, units=[(0, h) for h in range(w.n_kv_heads)])


# -- more than 4 query heads per kv head (head blocks) -----------------------------
@pytest.mark.parametrize("hq,hkv,d,bits,split", [
    (32, 1, 128, 2, 0), (32, 1, 128, 4, 0), (32, 1, 128, 2, 128), (16, 2, 128, 2, 0),
    (12, 1, 64, 8, 0), (71, 1, 64, 2, 0), (24, 2, 128, 4, 96),
])
def test_many_query_heads_per_kv_head(kvq, hq, hkv, d, bits, split):
    # MQA (one kv head for 32 query heads; Falcon-7B's 71 heads of d64 over
    # one kv head) and GQA above 4: head blocks of 4 query heads per
    # workgroup, also through the partial-state merge (forced splits)
    w = SMALL.scaled(n_q_heads=hq, n_kv_heads=hkv, d_h=d, bits=bits, group=32, residual=64,
                     context=900, batch=2, n_outlier=3, outlier_factor=8.0)
    run_kivi(kvq, w, units=[(b, h) for b in range(2) for h in range(hkv)], split_tokens=split)


def test_one_call_steps_mqa(kvq):
    # kvq_kivi_step with 32 query heads per kv head (eight head blocks): the
    # fused launch, every block's last wave writing the same append bytes
    # before it reads them, checked after every step
    w = SMALL.scaled(context=40, d_h=128, bits=2, group=32, residual=32, n_kv_heads=1, n_q_heads=32)
    launches = []
    run_kivi(kvq, w, units=[(0, 0)], steps=70, check_every_step=True, one_call=True, launches=launches)
    assert 1 in launches
    assert max(launches) >= 3                        # flush steps


# -- value magnitudes: large scale and outlier channels ------------------------------
@pytest.mark.parametrize("bits", [2, 4, 8])
def test_large_values_and_value_outliers(kvq, bits):
    # values N(0, 16^2) with three channels x2 more: the value loop's fp16
    # (offset + code) unpack, its fp16 weights p and p*s and the offset
    # removal after fp32 accumulation stay within the tolerance at large
    # magnitudes (a CPU emulation of the fp16 weights puts this case at about
    # 0.7 of the tolerance; the error grows with |V|, see the value-path
    # precision notes)
    w = SMALL.scaled(d_h=128, bits=bits, group=32, residual=64, context=1500, n_kv_heads=2, n_q_heads=4,
                     value_scale=16.0, n_value_outlier=3, value_outlier_factor=2.0, n_outlier=3,
                     outlier_factor=8.0)
    worst = run_kivi(kvq, w, units=[(0, 0), (0, 1)])
    print(f"int{bits} large values: max |gpu - oracle| = {worst:.3e}", flush=True)
