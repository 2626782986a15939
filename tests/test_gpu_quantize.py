"""GPU parity of kvq_quantize_append against the oracle: codes, scales and
zero points bit-exact, packed in the header's layout."""
import numpy as np
import pytest

from tests.helpers import ensure_built
from oracle import pack
from oracle.quant import quantize_keys, quantize_values

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvq():
    ensure_built()
    import decode_attention_kivi_amd as m
    return m


def _ties(n_streams, n, d):
    """Every key group (G tokens of a channel) and value group (G channels of
    a token) holds 0 and 3, so 2-bit groups get s = 1 and the codes of the
    other entries land on, or one fp16 ulp beside, the rounding boundaries
    k + 1/2 (where the kernels' reciprocal shortcut defers to the division)."""
    h = np.float16
    up = lambda v: np.nextafter(h(v), h(9))
    dn = lambda v: np.nextafter(h(v), h(-9))
    pat = np.array([0, 3, 0.5, 1.5, 2.5, up(0.5), dn(1.5), up(2.5), 1, 2, 0.25, 2.75,
                    up(1.5), dn(0.5), dn(2.5), dn(3)], np.float16)
    t, c = np.meshgrid(np.arange(n), np.arange(d), indexing="ij")
    return np.broadcast_to(pat[(t + c) % pat.size], (n_streams, n, d)).copy()


def _data(rng, n_streams, n, d, kind="normal"):
    if kind == "ties":
        return _ties(n_streams, n, d)
    if kind == "tiny":
        # groups whose fp16 scale is subnormal (range below (2^b - 1) 2^-14),
        # where the kernels' reciprocal path must defer to the clamped
        # division, beside normal ones: key groups (a channel over G tokens)
        # of channels c % 3 != 0 and value groups (a token over G channels)
        # of odd tokens hold only values of about 3e-5, 1e-7 or 4e-8 (by
        # stream; the smaller ones give scales of a few subnormal ulps, whose
        # rounding pushes quotients past 2^b - 1)
        x = rng.standard_normal((n_streams, n, d)).astype(np.float32)
        x *= np.array([3e-5, 1e-7, 4e-8], np.float32)[np.arange(n_streams) % 3][:, None, None]
        t, c = np.meshgrid(np.arange(n), np.arange(d), indexing="ij")
        x = np.where((c % 3 == 0) & (t % 2 == 0), rng.standard_normal((n_streams, n, d)), x)
        return x.astype(np.float16)
    x = rng.standard_normal((n_streams, n, d)).astype(np.float32)
    x[:, :, rng.choice(d, 3, replace=False)] *= 9.0
    if kind == "special":
        x[:, : min(n, 40), :16] = 0.5                  # constant groups: scale 0
        x[:, :, 20] = -0.0                             # negative zeros
        x[0, 3, :] = 1e-6                              # subnormal-range values
    return x.astype(np.float16)


def _run(kvq, which, bits, G, d, n_tok, dst_tok, gather, kind="normal", seed=0, S=3):
    import torch
    rng = np.random.default_rng([seed, which, bits, G, d, n_tok, dst_tok, S])
    n_src = n_tok + 5
    x = _data(rng, S, n_src, d, kind)
    rows = rng.permutation(n_src)[:n_tok].astype(np.int32) if gather else np.arange(n_tok, dtype=np.int32)
    total = dst_tok + n_tok
    if which == kvq.KVQ_KEYS:
        cb, mb = total * d * bits // 8, total // G * d * 4
    else:
        cb, mb = (total + 1) // 2 * d * bits // 4, (total + 1) // 2 * (d // G) * 8
    cb, mb = (cb + 15) // 16 * 16, (mb + 15) // 16 * 16
    dev = torch.device("cuda")
    xt = torch.from_numpy(x).to(dev)
    codes = torch.zeros(S, cb, dtype=torch.uint8, device=dev)
    meta = torch.zeros(S, mb, dtype=torch.uint8, device=dev)
    rt = torch.from_numpy(rows).to(dev) if gather else None
    print(f"quantize which={which} bits={bits} G={G} d={d} n={n_tok} dst={dst_tok} gather={gather} S={S}",
          flush=True)
    kvq.kvq_quantize_append(which, bits, G, S, d, n_tok, xt, n_src * d, d, rt, codes, cb, meta, mb, dst_tok)
    torch.cuda.synchronize()
    got_c, got_m = codes.cpu().numpy(), meta.cpu().numpy()
    for s in range(S):
        src = x[s][rows]
        if which == kvq.KVQ_KEYS:
            c, sc, z = quantize_keys(src, bits, G)
            full = np.zeros((total, d), np.uint8)
            full[dst_tok:] = c
            exp_c = pack.pack_rows(full, bits).reshape(-1)
            ms, mz = np.zeros((total // G, d), np.float16), np.zeros((total // G, d), np.float16)
            ms[dst_tok // G:], mz[dst_tok // G:] = sc, z
            exp_m = pack.pack_key_meta(ms, mz).view(np.uint8)
        else:
            c, sc, z = quantize_values(src, bits, G)
            full = np.zeros((total, d), np.uint8)
            full[dst_tok:] = c
            exp_c = pack.pack_values(full, bits).reshape(-1)
            ms, mz = np.zeros((total, d // G), np.float16), np.zeros((total, d // G), np.float16)
            ms[dst_tok:], mz[dst_tok:] = sc, z
            exp_m = pack.pack_value_meta(ms, mz).view(np.uint8)
        assert np.array_equal(got_c[s, :exp_c.size], exp_c), f"codes differ (stream {s})"
        assert not got_c[s, exp_c.size:].any()
        assert np.array_equal(got_m[s, :exp_m.size], exp_m), f"scale/zero differ (stream {s})"
        assert not got_m[s, exp_m.size:].any()


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [32, 64, 128])
def test_keys_bit_exact(kvq, bits, d, G):
    _run(kvq, kvq.KVQ_KEYS, bits, G, d, n_tok=2 * G, dst_tok=G, gather=False)


@pytest.mark.parametrize("bits,d,G,gather", [(2, 128, 32, False), (8, 64, 64, True)])
def test_keys_many_streams(kvq, bits, d, G, gather):
    """8192 key groups in one launch (256 streams x 32 groups)."""
    _run(kvq, kvq.KVQ_KEYS, bits, G, d, n_tok=32 * G, dst_tok=G, gather=gather, S=256)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("d,G", [(64, 32), (64, 64), (128, 32), (128, 64), (128, 128)])
def test_values_bit_exact_odd_offsets(kvq, bits, d, G):
    _run(kvq, kvq.KVQ_VALUES, bits, G, d, n_tok=37, dst_tok=5, gather=False)
    _run(kvq, kvq.KVQ_VALUES, bits, G, d, n_tok=1, dst_tok=0, gather=False)


@pytest.mark.parametrize("which", [0, 1])
@pytest.mark.parametrize("bits", [2, 4, 8])
def test_gather_and_special_values(kvq, which, bits):
    _run(kvq, which, bits, 32, 128, n_tok=96, dst_tok=0, gather=True, kind="special")


@pytest.mark.parametrize("which", [0, 1])
@pytest.mark.parametrize("bits", [2, 4, 8])
def test_codes_on_rounding_boundaries(kvq, which, bits):
    _run(kvq, which, bits, 32, 128, n_tok=96, dst_tok=0, gather=False, kind="ties")


@pytest.mark.parametrize("which", [0, 1])
@pytest.mark.parametrize("bits", [2, 4, 8])
def test_subnormal_scales(kvq, which, bits):
    _run(kvq, which, bits, 32, 128, n_tok=96, dst_tok=0, gather=False, kind="tiny")
    _run(kvq, which, bits, 64, 64, n_tok=128, dst_tok=64 if which == 0 else 3, gather=False, kind="tiny")


@pytest.mark.parametrize("which", [0, 1])
def test_two_runs_bit_identical(kvq, which):
    """Determinism: quantizing the same rows twice gives the same bytes."""
    import torch
    rng = np.random.default_rng([12, which])
    S, n, d, G = 4, 256, 128, 32
    x = torch.from_numpy(_data(rng, S, n, d)).cuda()
    outs = []
    for _ in range(2):
        codes = torch.zeros(S, n * d, dtype=torch.uint8, device="cuda")
        meta = torch.zeros(S, n * d, dtype=torch.uint8, device="cuda")
        print(f"quantize determinism which={which}", flush=True)
        kvq.kvq_quantize_append(which, 2, G, S, d, n, x, n * d, d, None, codes, n * d, meta, n * d, 0)
        torch.cuda.synchronize()
        outs.append((codes.cpu().numpy(), meta.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


def test_fp16_run_is_a_copy(kvq):
    import torch
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 40, 64)).astype(np.float16)
    rows = rng.permutation(40)[:32].astype(np.int32)
    dev = torch.device("cuda")
    out = torch.zeros(2, 48 * 64 * 2, dtype=torch.uint8, device=dev)
    print("quantize bits=16 copy", flush=True)
    kvq.kvq_quantize_append(kvq.KVQ_VALUES, 16, 32, 2, 64, 32, torch.from_numpy(x).to(dev), 40 * 64,
                            64, torch.from_numpy(rows).to(dev), out, out.stride(0), None, 0, 16)
    got = out.cpu().numpy().view(np.float16).reshape(2, 48, 64)
    assert np.array_equal(got[:, 16:], x[:, rows]) and not got[:, :16].view(np.uint16).any()


# -- kvq_decode_append: one step's residual/window rows plus one value token ---------
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("d,G", [(64, 32), (128, 32), (128, 64)])
@pytest.mark.parametrize("dst_tok,quant", [(6, "old"), (7, "old"), (7, "new"), (5, "none")])
def test_decode_append_bit_exact(kvq, bits, d, G, dst_tok, quant):
    import torch
    rng = np.random.default_rng([7, bits, d, G, dst_tok, len(quant)])
    S, R_rows, K_rows = 3, 6, 4
    dev = torch.device("cuda")
    k_new = _data(rng, S, 1, d)[:, 0]
    v_new = _data(rng, S, 1, d)[:, 0]
    v_win = _data(rng, S, R_rows, d)
    k_res0 = _data(rng, S, K_rows, d)
    # a value run that already holds dst_tok tokens (oracle bytes)
    old = _data(rng, S, dst_tok, d)
    k_row, v_row = 2, 4
    v_quant_row = {"old": 1, "new": v_row, "none": -1}[quant]
    total = dst_tok + 1
    cb = ((total + 1) // 2 * d * bits // 4 + 15) // 16 * 16
    mb = ((total + 1) // 2 * (d // G) * 8 + 15) // 16 * 16
    codes0 = np.zeros((S, cb), np.uint8)
    meta0 = np.zeros((S, mb), np.uint8)
    for s in range(S):
        c, sc, z = quantize_values(old[s], bits, G)
        e = pack.pack_values(c, bits).reshape(-1)
        codes0[s, :e.size] = e
        m = pack.pack_value_meta(sc, z).view(np.uint8)
        meta0[s, :m.size] = m
    kn, vn = torch.from_numpy(k_new).to(dev), torch.from_numpy(v_new).to(dev)
    kr, vr = torch.from_numpy(k_res0.copy()).to(dev), torch.from_numpy(v_win.copy()).to(dev)
    codes, meta = torch.from_numpy(codes0).to(dev), torch.from_numpy(meta0).to(dev)
    print(f"decode_append bits={bits} d={d} G={G} dst={dst_tok} quant={quant}", flush=True)
    kvq.kvq_decode_append(bits, G, S, d, kn, d, vn, d, kr, K_rows * d, k_row, vr, R_rows * d, v_row,
                          v_quant_row, codes, cb, meta, mb, dst_tok)
    torch.cuda.synchronize()
    exp_k = k_res0.copy()
    exp_k[:, k_row] = k_new
    exp_v = v_win.copy()
    exp_v[:, v_row] = v_new
    assert np.array_equal(kr.cpu().numpy().view(np.uint16), exp_k.view(np.uint16))
    assert np.array_equal(vr.cpu().numpy().view(np.uint16), exp_v.view(np.uint16))
    got_c, got_m = codes.cpu().numpy(), meta.cpu().numpy()
    for s in range(S):
        if quant == "none":
            exp_c, exp_m = codes0[s], meta0[s]
        else:
            toks = np.concatenate([old[s], exp_v[s, v_quant_row][None]], axis=0)
            c, sc, z = quantize_values(toks, bits, G)
            exp_c = np.zeros(cb, np.uint8)
            e = pack.pack_values(c, bits).reshape(-1)
            exp_c[:e.size] = e
            exp_m = np.zeros(mb, np.uint8)
            m = pack.pack_value_meta(sc, z).view(np.uint8)
            exp_m[:m.size] = m
        assert np.array_equal(got_c[s], exp_c), f"value codes differ (stream {s})"
        assert np.array_equal(got_m[s], exp_m), f"value scale/zero differ (stream {s})"
