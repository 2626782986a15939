"""The quantizer kernels' shortcut for the correctly rounded division
(kvq_quant.h, encode_fast): q0 = fl(d * r) with r within 1 ulp of 1/s, and
the exact division only when q0 lies within 2^b * 2^-20 of a half-integer.
Emulated here in float32 against the plain definition clamp(rint(fl(d / s)))
over every positive finite fp16 scale, with quotients placed on, just
around and far from the rounding boundaries, and r taken 1 ulp low, exact
and 1 ulp high.  No GPU: this checks the argument the kernels rely on."""
import numpy as np

F32 = np.float32


def _fast(d, s, r, qmax):
    q = (d * r).astype(F32)
    t = np.rint(q)
    slow = np.abs((q - t).astype(F32)) >= F32(0.5 - (qmax + 1) * 2.0 ** -20)
    q = np.where(slow, (d / s).astype(F32), q)
    return np.clip(np.rint(q), 0, qmax), slow


def _exact(d, s, qmax):
    return np.clip(np.rint((d / s).astype(F32)), 0, qmax)


def test_every_fp16_scale_near_every_boundary():
    s16 = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16)       # positive finite fp16
    s = s16.astype(F32)
    rng = np.random.default_rng(3)
    slow_total = 0
    n_total = 0
    for bits in (2, 4, 8):
        qmax = (1 << bits) - 1
        # targets: every rounding boundary k + 1/2 inside the code range, a
        # few integers and random interior points
        ks = np.arange(0, qmax + 1)
        targets = np.concatenate([ks + 0.5, ks.astype(np.float64), rng.uniform(-1, qmax + 1, 8)])
        for t in targets:
            base = (F32(t) * s).astype(F32)                   # d with d / s close to t
            for ulps in (-3, -1, 0, 1, 3):
                d = np.nextafter(base, np.where(ulps < 0, -np.inf, np.inf).astype(F32)) if ulps else base
                for _ in range(abs(ulps) - 1 if abs(ulps) > 1 else 0):
                    d = np.nextafter(d, F32(np.inf) if ulps > 0 else F32(-np.inf))
                d = d.astype(F32)
                ok = np.isfinite(d)
                for rdir in (-1, 0, 1):
                    r = (F32(1) / s).astype(F32)
                    if rdir:
                        r = np.nextafter(r, F32(np.inf) if rdir > 0 else F32(0)).astype(F32)
                    got, slow = _fast(d[ok], s[ok], r[ok], qmax)
                    want = _exact(d[ok], s[ok], qmax)
                    assert np.array_equal(got, want), (bits, t, ulps, rdir)
                    slow_total += int(slow.sum())
                    n_total += int(ok.sum())
    # the exact division is the exception, not the rule, even on these
    # boundary-heavy inputs
    assert slow_total < n_total // 2


def test_random_groups_rarely_take_the_division():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((4096, 32)).astype(np.float16).astype(F32)
    for bits in (2, 4, 8):
        qmax = (1 << bits) - 1
        mn, mx = x.min(1, keepdims=True), x.max(1, keepdims=True)
        s = np.float16((mx - mn) / F32(qmax)).astype(F32)
        z = np.float16(mn).astype(F32)
        d = (x - z).astype(F32)
        r = (F32(1) / s).astype(F32)
        got, slow = _fast(d, s, r, qmax)
        assert np.array_equal(got, _exact(d, s, qmax))
        assert slow.mean() < 1e-3


def test_normal_scales_need_no_clamp():
    """The row-batch encoder (codes8_fast) drops the clamp for groups whose
    fp16 scale s = fl16(fl32(D / (2^b - 1))), D = fl32(max - min), is normal:
    d = fl32(x - z) <= D with z = min exactly, so the largest product is
    fl32(D * r) at the largest D that still rounds to s, with r one ulp above
    1/s; its rint must not pass 2^b - 1.  Checked for every normal fp16 s."""
    s16 = np.arange(0x0400, 0x7C00, dtype=np.uint16)
    s = s16.view(np.float16).astype(F32)
    nxt = (s16 + 1).view(np.float16).astype(np.float64)          # next fp16 (inf past the last)
    nxt[-1] = 65520.0                                             # the fp16 overflow threshold
    for bits in (2, 4, 8):
        qmax = (1 << bits) - 1
        hi = ((s.astype(np.float64) + nxt) / 2 * qmax).astype(F32)  # about the largest D for s
        worst = np.zeros_like(s)
        for k in range(-6, 7):                                   # fp32 values around it
            D = hi.copy()
            for _ in range(abs(k)):
                D = np.nextafter(D, F32(np.inf) if k > 0 else F32(0)).astype(F32)
            maps = np.float16((D / F32(qmax)).astype(F32)) == s16.view(np.float16)
            r = np.nextafter((F32(1) / s).astype(F32), F32(np.inf)).astype(F32)
            q = (D * r).astype(F32)
            worst = np.where(maps & (q > worst), q, worst)
        assert (worst > 0).all()
        assert np.rint(worst).max() <= qmax, bits
        assert (worst < qmax + 0.25).all()
