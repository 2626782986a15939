"""The C-ABI library loads, exports every symbol include/kvq.h declares, and
rejects bad arguments on the host with the documented status codes (before
any HIP call, so these run without a GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

from tests.helpers import ROOT, ensure_built

ensure_built()
import decode_attention_kivi_amd as kvq  # noqa: E402
from decode_attention_kivi_amd import KVQ_KEYS, KVQ_VALUES, KvqError  # noqa: E402

EINVAL, EALIGN, EUNSUP, EWS, ESCRATCH = 1, 2, 3, 4, 6
A = 1 << 20        # a fake, 16-byte aligned device address (never dereferenced)


def declared_functions():
    text = open(os.path.join(ROOT, "include", "kvq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = ctypes.CDLL(kvq.library_path())
    names = declared_functions()
    assert {"kvq_quantize_append", "kvq_reorder_windows", "kvq_decode_attn"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strings():
    assert kvq.kvq_abi_version() == 1
    assert kvq.kvq_strerror(0) == "ok"
    assert "workspace" in kvq.kvq_strerror(4)
    assert kvq.kvq_strerror(99) == "unknown status"


def _q(**kw):
    args = dict(which=KVQ_KEYS, bits=2, group=32, n_streams=2, d_h=128, n_tok=64, src=A,
                src_stream_stride=128 * 64, src_row_stride=128, src_rows=None, codes=A,
                codes_stream_stride=4096, meta=A, meta_stream_stride=4096, dst_tok=0, stream=0)
    args.update(kw)
    return kvq.kvq_quantize_append(**args)


@pytest.mark.parametrize("kw,code", [
    (dict(which=7), EINVAL), (dict(bits=3), EINVAL), (dict(group=16), EUNSUP),
    (dict(d_h=96), EUNSUP), (dict(n_tok=33), EINVAL), (dict(dst_tok=16), EINVAL),
    (dict(src=None), EINVAL), (dict(meta=None), EINVAL), (dict(src=A + 2), EALIGN),
    (dict(codes=A + 8), EALIGN), (dict(src_row_stride=132), EALIGN),
    (dict(src_row_stride=64), EINVAL), (dict(codes_stream_stride=4100), EALIGN),
    (dict(n_streams=0), EINVAL), (dict(n_streams=70000), EUNSUP),
    (dict(which=KVQ_VALUES, group=128, d_h=64), EUNSUP),
])
def test_quantize_rejects(kw, code):
    with pytest.raises(KvqError) as e:
        _q(**kw)
    assert e.value.status == code


def test_quantize_empty_is_a_noop():
    _q(n_tok=0)                      # returns OK without launching anything
    _q(which=KVQ_VALUES, n_tok=0, dst_tok=3)


@pytest.mark.parametrize("kw,code", [
    (dict(d_h=32), EUNSUP), (dict(n_rows=-1), EINVAL), (dict(dst=A + 4), EALIGN),
    (dict(src_stream_stride=12), EALIGN), (dict(src=None), EINVAL),
])
def test_residual_append_rejects(kw, code):
    args = dict(n_streams=2, d_h=64, n_rows=1, src=A, src_stream_stride=64, src_row_stride=64,
                dst=A, dst_stream_stride=64 * 8, dst_row=0, stream=0)
    args.update(kw)
    with pytest.raises(KvqError) as e:
        kvq.kvq_residual_append(**args)
    assert e.value.status == code


@pytest.mark.parametrize("kw,code", [
    (dict(n_windows=0), EINVAL), (dict(n_windows=70000), EINVAL), (dict(window_tokens=48), EINVAL),
    (dict(group=16), EUNSUP), (dict(perm=None), EINVAL), (dict(perm=A + 2), EALIGN),
])
def test_reorder_rejects(kw, code):
    args = dict(win_bits=A, n_windows=8, window_tokens=64, group=32, d_h=128, perm=A, segs=A,
                n_segs=A, row_gather=None, stream=0)
    args.update(kw)
    with pytest.raises(KvqError) as e:
        kvq.kvq_reorder_windows(**args)
    assert e.value.status == code


def _decode(**kw):
    base = dict(batch=2, n_q_heads=8, n_kv_heads=2, d_h=128, group=32, sm_scale=0.0884, q=A,
                k_segs=[(2, 0, 256, 0, 0)], v_segs=[(2, 0, 200, 0, 0)],
                k_codes=A, k_codes_stride=1 << 16, k_meta=A, k_meta_stride=1 << 16,
                v_codes=A, v_codes_stride=1 << 16, v_meta=A, v_meta_stride=1 << 16,
                k_res=A, n_k_res=3, k_res_stride=128 * 128, v_res=A, n_v_res=59,
                v_res_stride=128 * 128, out=A, split_tokens=64)
    base.update(kw)
    return kvq.make_decode_args(**base)


def test_workspace_size_follows_the_split_plan():
    a = _decode()
    # N = 256 + 3 = 259 tokens, 64 per workgroup: 5 workgroups per stream;
    # workspace = partial states, streams * workgroups * gq * (d + 2) floats
    assert kvq.kvq_decode_attn_workspace(a) == 2 * 2 * 5 * 4 * 130 * 4
    # one workgroup per stream writes the output directly: no workspace
    assert kvq.kvq_decode_attn_workspace(_decode(split_tokens=512)) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(n_q_heads=7), EINVAL), (dict(n_q_heads=2 * 16 + 1), EINVAL), (dict(d_h=96), EUNSUP),
    (dict(n_k_res=4), EINVAL), (dict(k_segs=[(2, 0, 250, 0, 0)], n_k_res=9), EINVAL),
    (dict(k_segs=[(3, 0, 256, 0, 0)]), EINVAL), (dict(k_segs=[(2, 0, 256, 8, 0)]), EALIGN),
    (dict(v_segs=[(2, 5, 200, 0, 0)]), EINVAL), (dict(q=A + 2), EALIGN),
    (dict(k_codes_stride=100), EALIGN), (dict(k_res_stride=12), EALIGN),
    (dict(sm_scale=float("nan")), EINVAL), (dict(k_codes=None), EINVAL),
    # one forced workgroup for 8195 tokens: waves of ~1024 tokens exceed the cap
    (dict(k_segs=[(2, 0, 8192, 0, 0)], v_segs=[(2, 0, 8136, 0, 0)], split_tokens=1 << 20), EUNSUP),
    (dict(group=128, d_h=64), EUNSUP),
    # a quantized key run must start on a group boundary, a quantized value run on a pair
    (dict(k_segs=[(16, 0, 16, 0, 0), (2, 16, 256, 4096, 0)], v_segs=[(2, 0, 216, 0, 0)]), EUNSUP),
    (dict(v_segs=[(16, 0, 11, 0, 0), (2, 11, 189, 4096, 0)]), EUNSUP),
])
def test_decode_rejects(kw, code):
    with pytest.raises(KvqError) as e:
        kvq.kvq_decode_attn_workspace(_decode(**kw))
    assert e.value.status == code


def test_decode_needs_workspace():
    a = _decode()
    with pytest.raises(KvqError) as e:
        kvq.kvq_decode_attn(a, 0)
    assert e.value.status == EWS
    a.workspace = A
    a.workspace_bytes = kvq.kvq_decode_attn_workspace(a) - 4
    with pytest.raises(KvqError) as e:
        kvq.kvq_decode_attn(a, 0)
    assert e.value.status == EWS


@pytest.mark.parametrize("hq,hkv", [(32, 1), (16, 2), (12, 1), (64, 4)])
def test_any_head_ratio_plans(hq, hkv):
    """More than 4 query heads per kv head run in head blocks of 4 (one more
    grid dimension); the partial states still cover every query head."""
    a = _decode(batch=2, n_q_heads=hq, n_kv_heads=hkv)
    # N = 259, 64 tokens per workgroup: 5 workgroups per stream
    assert kvq.kvq_decode_attn_workspace(a) == 2 * hkv * 5 * (hq // hkv) * 130 * 4


def test_noalloc_checks_before_any_launch():
    """kvq_decode_attn_noalloc applies kvq_decode_attn's checks and refuses a
    plan whose partial states exceed the static scratch (KVQ_ESCRATCH),
    all on the host: nothing here is launched."""
    with pytest.raises(KvqError) as e:
        kvq.kvq_decode_attn_noalloc(_decode(n_q_heads=7), 0)
    assert e.value.status == EINVAL
    big = _decode(batch=64, n_q_heads=64, n_kv_heads=8, k_segs=[(2, 0, 8192, 0, 0)],
                  v_segs=[(2, 0, 8136, 0, 0)], split_tokens=64)
    assert kvq.kvq_decode_attn_workspace(big) > kvq.KVQ_SCRATCH_BYTES
    with pytest.raises(KvqError) as e:
        kvq.kvq_decode_attn_noalloc(big, 0)
    assert e.value.status == ESCRATCH
    assert "scratch" in kvq.kvq_strerror(ESCRATCH)


def test_binding_refuses_host_tensors_as_device_buffers():
    import torch
    with pytest.raises(ValueError):
        _q(src=torch.zeros(16, dtype=torch.float16))


def _kivi(**kw):
    base = dict(bits=2, group=32, residual=64, n_streams=4, d_h=128, capacity=1024, win_rows=130,
                reserved=0, k_codes=A, k_codes_stride=1 << 16, k_meta=A, k_meta_stride=1 << 16,
                v_codes=A, v_codes_stride=1 << 16, v_meta=A, v_meta_stride=1 << 16,
                k_res=A, k_res_stride=64 * 128, v_res=A, v_res_stride=130 * 128,
                n_kq=256, r_k=5, n_vq=197, r_v=64, v_start=3)
    base.update(kw)
    return kvq.KiviCacheDesc(**base)


def test_kivi_step_workspace_follows_the_state_after_the_step():
    # 262 tokens after the step, one workgroup per stream: no workspace
    assert kvq.kvq_kivi_step_workspace(_kivi(), 2, 8) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(bits=3), EINVAL), (dict(group=16), EINVAL), (dict(d_h=96), EUNSUP),
    (dict(residual=48), EINVAL), (dict(win_rows=129), EINVAL), (dict(reserved=1), EINVAL),
    (dict(r_k=64), EINVAL), (dict(n_kq=250), EINVAL), (dict(r_v=65, n_vq=196), EINVAL),
    (dict(n_vq=198), EINVAL),                    # token counts of keys and values differ
    (dict(v_start=67), EINVAL),                  # window past the ring
    (dict(capacity=261), EINVAL),                # no room for the new token
    (dict(n_streams=5), EINVAL),                 # not batch * n_kv_heads
])
def test_kivi_step_rejects(kw, code):
    with pytest.raises(KvqError) as e:
        kvq.kvq_kivi_step_workspace(_kivi(**kw), 2, 8)
    assert e.value.status == code


def test_kivi_step_rejects_before_any_launch_and_keeps_the_state():
    c = _kivi()
    for kw, code in [(dict(k_new=A + 2), EALIGN), (dict(q=None), EINVAL), (dict(n_q_heads=7), EINVAL),
                     (dict(k_new_stride=64), EINVAL)]:
        args = dict(batch=2, n_q_heads=8, sm_scale=0.088, k_new=A, k_new_stride=128, v_new=A,
                    v_new_stride=128, q=A, out=A, workspace=None, workspace_bytes=0, stream=0)
        args.update(kw)
        with pytest.raises(KvqError) as e:
            kvq.kvq_kivi_step(c, **args)
        assert e.value.status == code
        assert (c.n_kq, c.r_k, c.n_vq, c.r_v, c.v_start) == (256, 5, 197, 64, 3)


def test_window_thresholds_host_values():
    lo, hi = kvq.kvq_window_thresholds(0.5, 2.0)
    assert abs(lo - 0.2689414213699951) < 1e-7 and abs(hi - 0.7310585786300049) < 1e-7
    for bad in [(0.5, 0.0), (float("nan"), 2.0), (0.5, float("inf"))]:
        with pytest.raises(KvqError) as e:
            kvq.kvq_window_thresholds(*bad)
        assert e.value.status == EINVAL


def test_window_search_workspace_is_chunk_sums():
    # 4 windows of 100 tokens -> 2 chunks each; 70 text tokens -> 2 chunks
    assert kvq.kvq_window_search_workspace(3, 70, 405, 64, 100) == 3 * (4 * 2 + 2) * 64 * 4


def _search(**kw):
    base = dict(batch=2, n_text=16, n_visual=512, dim=128, text=A, text_batch_stride=16 * 128,
                text_row_stride=128, visual=A, visual_batch_stride=512 * 128, visual_row_stride=128,
                window_tokens=64, t_low=0.3, t_high=0.7, first_window_fp16=1, scores=None,
                win_bits=A, workspace=A, workspace_bytes=1 << 30, stream=0)
    base.update(kw)
    return base


@pytest.mark.parametrize("kw,code", [
    (dict(dim=12), EINVAL), (dict(dim=8192), EUNSUP), (dict(n_visual=63), EINVAL),
    (dict(n_text=0), EINVAL), (dict(batch=0), EINVAL), (dict(window_tokens=0), EINVAL),
    (dict(text_row_stride=120), EINVAL), (dict(visual_row_stride=132), EALIGN),
    (dict(text=A + 8), EALIGN), (dict(scores=A + 2), EALIGN), (dict(win_bits=None), EINVAL),
    (dict(t_low=float("nan")), EINVAL), (dict(workspace_bytes=100), EWS), (dict(workspace=None), EWS),
])
def test_window_search_rejects(kw, code):
    with pytest.raises(KvqError) as e:
        kvq.kvq_window_search(**_search(**kw))
    assert e.value.status == code


# --- paged, ragged cache -----------------------------------------------------

@pytest.mark.parametrize("H,d,G,bits,PT", [(32, 128, 32, 2, 256), (2, 64, 64, 4, 64), (8, 128, 128, 8, 128)])
def test_page_layout_is_a_key_run_and_a_value_run(H, d, G, bits, PT):
    # a head block = PT key rows, PT/G key groups of (scale, zero) pairs,
    # PT/2 value pair blocks, PT * d/G value pairs (the run formats)
    L = kvq.kvq_page_layout(H, d, G, bits, PT)
    rb = d * bits // 8
    assert L["kmeta_off"] == PT * rb
    assert L["vcodes_off"] == PT * rb + (PT // G) * d * 4
    assert L["vmeta_off"] == L["vcodes_off"] + (PT // 2) * 2 * rb
    assert L["head_bytes"] == L["vmeta_off"] + PT * (d // G) * 4
    assert L["page_bytes"] == H * L["head_bytes"] and L["page_bytes"] % 16 == 0


@pytest.mark.parametrize("kw,code", [
    (dict(PT=96), EUNSUP), (dict(PT=64, G=128), EUNSUP), (dict(bits=16), EINVAL),
    (dict(G=128, d=64), EUNSUP), (dict(H=0), EINVAL),
])
def test_page_layout_rejects(kw, code):
    a = dict(H=4, d=128, G=32, bits=2, PT=256)
    a.update(kw)
    with pytest.raises(KvqError) as e:
        kvq.kvq_page_layout(a["H"], a["d"], a["G"], a["bits"], a["PT"])
    assert e.value.status == code


def _paged(lengths, **kw):
    """kvq_decode_attn_paged with fake device pointers (the host checks only)."""
    import numpy as np
    lens = np.asarray(lengths, dtype=np.int32).reshape(-1, 4)
    a = kvq.PagedArgs()
    a.batch, a.n_q_heads, a.n_kv_heads, a.d_h, a.group, a.bits = len(lens), 4, 2, 128, 32, 2
    a.sm_scale, a.page_tokens = 0.088, 256
    a.q = a.pages = a.block_table = a.lengths_dev = a.k_res = a.v_res = a.out = A
    a.page_bytes = kvq.kvq_page_layout(2, 128, 32, 2, 256)["page_bytes"]
    a.max_pages = 4
    a.lengths = lens.ctypes.data
    a.k_res_stride = a.v_res_stride = 129 * 128
    for k, v in kw.items():
        setattr(a, k, v)
    return a, lens


def test_paged_workspace_sizes():
    # (n_kq, n_vq, n_k_res, n_v_res); one workgroup per stream -> no workspace
    a, lens = _paged([[512, 385, 1, 128], [0, 0, 5, 5]])
    assert kvq.kvq_decode_attn_paged_workspace(a) == 0
    # with 2 query heads per kv head an 8-wave workgroup covers 8 * 768
    # tokens of 2-bit keys and values (96 bytes each; waves up to the LDS
    # cap of 800 slots less the 32-token alignment): 5000 such tokens plus
    # 120 residual-value tokens (304 bytes) fit one, 6024 plus 120 need two:
    # the workspace holds B * Hkv * 2 partial states of gq * (d + 2) floats
    a, lens = _paged([[5120, 5000, 0, 120], [32, 0, 0, 32]], max_pages=20)
    assert kvq.kvq_decode_attn_paged_workspace(a) == 0
    a, lens = _paged([[6144, 6024, 0, 120], [32, 0, 0, 32]], max_pages=24)
    assert kvq.kvq_decode_attn_paged_workspace(a) == 2 * 2 * 2 * 2 * 130 * 4
    a.workspace, a.workspace_bytes = A, 100
    with pytest.raises(KvqError) as e:
        kvq.kvq_decode_attn_paged(a, 0)
    assert e.value.status == EWS


@pytest.mark.parametrize("lengths,kw,code", [
    ([[33, 0, 0, 33]], {}, EINVAL),                 # n_kq not whole key groups
    ([[64, 65, 0, -1]], {}, EINVAL),                # n_vq > n_kq
    ([[64, 0, 1, 64]], {}, EINVAL),                 # key and value totals differ
    ([[0, 0, 0, 0]], {}, EINVAL),                   # no token at all
    ([[1280, 1280, 0, 0]], {}, EINVAL),             # 5 pages > max_pages
    ([[64, 64, 0, 0]], dict(page_bytes=16), EINVAL),
    ([[64, 64, 0, 0]], dict(page_bytes=24576 * 2 + 8), EALIGN),
    ([[64, 64, 0, 0]], dict(pages=A + 4), EALIGN),
    ([[64, 64, 0, 0]], dict(block_table=A + 2), EALIGN),
    ([[64, 64, 0, 0]], dict(k_res_stride=12), EALIGN),
    ([[64, 64, 0, 0]], dict(lengths_dev=None), EINVAL),
    ([[64, 64, 0, 0]], dict(n_q_heads=37, n_kv_heads=2), EINVAL),
    ([[64, 64, 0, 0]], dict(page_tokens=100), EUNSUP),
    ([[64, 32, 0, 32]], dict(v_res=None), EINVAL),  # value residual rows but no buffer
])
def test_paged_rejects(lengths, kw, code):
    a, lens = _paged(lengths, **kw)
    with pytest.raises(KvqError) as e:
        kvq.kvq_decode_attn_paged(a, 0)
    assert e.value.status == code


def test_split_plan_fills_the_chip_once():
    # GQA long context (4 sequences, 32 q / 8 kv heads, 32769 tokens, G64):
    # 32 streams of 4 query heads run one 12-wave workgroup per CU with waves
    # of up to 512 tokens; 8 workgroups per stream (256 = one round over 256
    # CUs) beat 9 to 16 (two rounds) -- workspace = 32 * 8 partial states
    a = _decode(batch=4, n_q_heads=32, n_kv_heads=8, group=64, k_segs=[(2, 0, 32768, 0, 0)],
                v_segs=[(2, 0, 32641, 0, 0)], n_k_res=1, n_v_res=128, split_tokens=0)
    assert kvq.kvq_decode_attn_workspace(a) == 32 * 8 * 4 * 130 * 4
    # one query head per kv head, 512 streams of 4097 tokens: one workgroup
    # per stream (two per CU) and no workspace
    a = _decode(batch=16, n_q_heads=32, n_kv_heads=32, k_segs=[(2, 0, 4096, 0, 0)],
                v_segs=[(2, 0, 3969, 0, 0)], n_k_res=1, n_v_res=128, split_tokens=0)
    assert kvq.kvq_decode_attn_workspace(a) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(m=3), EUNSUP), (dict(m=32), EUNSUP), (dict(d_h=96), EUNSUP), (dict(bits=9), EINVAL),
    (dict(bits=0), EINVAL), (dict(top_k=0), EINVAL), (dict(top_k=101), EINVAL), (dict(n_tok=0), EINVAL),
    (dict(codes_stride=192), EINVAL), (dict(codes_stride=204), EALIGN), (dict(q=A + 2), EALIGN),
    (dict(top_idx=A + 2), EALIGN), (dict(scores=None), EINVAL), (dict(n_q_heads=7), EINVAL),
    (dict(n_q_heads=4 * 16 + 2), EINVAL),
    # too many tokens for a head's scores in LDS, and the scores kernel's 8
    # query heads x 16 sub-spaces x 256 centroids of fp32 tables: 128 KB > 64 KB
    (dict(n_q_heads=32, m=16, n_tok=100000, codes_stride=1600000), EUNSUP),
])
def test_pq_search_rejects(kw, code):
    a = dict(batch=2, n_q_heads=4, n_kv_heads=4, d_h=128, m=2, bits=8, n_tok=100, top_k=10,
             q=A, centroids=A, codes=A, codes_stride=208, scores=A, top_idx=A, stream=0)
    a.update(kw)
    with pytest.raises(KvqError) as e:
        kvq.kvq_pq_search(**a)
    assert e.value.status == code


def test_vq_workspace_plan():
    # 512 streams (Llama-2-7B MHA shape, 4096 tokens): one chunk per stream,
    # no partial states
    assert kvq.kvq_vq_decode_attn_workspace(16, 32, 32, 128, 1, 4096) == 0
    # 32 streams of 32768 tokens (GQA long context): 16 chunks of 2048 tokens
    # fill 512 workgroups; partial states of 4 query heads per chunk
    assert kvq.kvq_vq_decode_attn_workspace(4, 32, 8, 128, 2, 32768) == 32 * 16 * 4 * 130 * 4
    # a short context is never cut below 256 tokens per chunk
    assert kvq.kvq_vq_decode_attn_workspace(1, 1, 1, 64, 1, 300) == 2 * 1 * 66 * 4


@pytest.mark.parametrize("kw,code", [
    (dict(d_h=96, codes_stride=2400), EUNSUP), (dict(rounds=3), EUNSUP), (dict(n_tok=0), EINVAL),
    (dict(n_q_heads=5), EINVAL), (dict(codes_stride=3184), EINVAL), (dict(codes_stride=3208), EALIGN),
    (dict(q=A + 2), EALIGN), (dict(k_books=A + 8), EALIGN), (dict(out=A + 2), EALIGN),
    (dict(v_codes=None), EINVAL), (dict(sm_scale=float("nan")), EINVAL),
    (dict(n_tok=1 << 25, codes_stride=1 << 30), EINVAL),
    (dict(batch=1, n_q_heads=1, n_kv_heads=1, workspace=None), EWS),   # 2 chunks need partial states
])
def test_vq_decode_rejects(kw, code):
    a = dict(batch=2, n_q_heads=4, n_kv_heads=2, d_h=128, rounds=1, n_tok=100, sm_scale=0.1, q=A, k_codes=A,
             v_codes=A, codes_stride=3200, k_books=A, v_books=A, out=A, workspace=A, workspace_bytes=1 << 20,
             stream=0)
    a.update(kw)
    if "n_tok" not in kw and a["batch"] == 1:
        a["n_tok"] = 300                 # one stream of 300 tokens: two chunks
        a["codes_stride"] = 300 * 32 // 16 * 16 + 16
    with pytest.raises(KvqError) as e:
        kvq.kvq_vq_decode_attn(**a)
    assert e.value.status == code


def test_vq_chunk_plan_properties():
    # chunks cover the context, hold at most 8192 tokens, are not cut below
    # 256 tokens (unless the context is shorter), and a split happens only
    # when the streams alone give fewer than 512 workgroups or the context
    # exceeds one chunk; the chunk count is read back from the workspace
    rng = np.random.default_rng(11)
    for _ in range(300):
        B = int(rng.integers(1, 40))
        hkv = int(rng.choice([1, 2, 4, 8, 32]))
        gq = int(rng.integers(1, 9))
        d = int(rng.choice([64, 128]))
        R = int(rng.integers(1, 3))
        n = int(rng.integers(1, 200000))
        ws = kvq.kvq_vq_decode_attn_workspace(B, hkv * gq, hkv, d, R, n)
        streams = B * hkv
        nc = 1 if ws == 0 else ws // (streams * gq * (d + 2) * 4)
        assert ws == 0 or ws == streams * nc * gq * (d + 2) * 4
        assert 1 <= nc <= 1024
        assert nc >= -(-n // 8192)
        if nc > 1:
            assert -(-n // nc) >= 64 and (n > 8192 or streams * nc <= 2 * 512)
        if n <= 256 and streams >= 1:
            assert nc == 1
