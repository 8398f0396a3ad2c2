"""The quantizer's reciprocal shortcut, checked on the CPU in NumPy float32 (no GPU, no
library): for the quotients w4_quantize forms, q = rint_even(RN(d / s)) with d = RN(w - lo)
and s = RN16(RN(hi - lo) / 15), the product a = RN(d * r) with r within 2 ulps of 1/s rounds
to the same integer whenever a is farther than 4e-5 from a half-integer, and a stays below
31.  The kernel divides exactly in the other cases; this test pins the bound it relies on."""

import numpy as np

F32 = np.float32


def _shortcut_mismatches(d, s):
    d, s = d.astype(F32), s.astype(F32)
    q = (d / s).astype(F32)                       # correctly rounded float32 quotient
    r0 = (F32(1.0) / s).astype(F32)
    bad = 0
    for k in (-2, -1, 0, 1, 2):                   # a reciprocal off by up to 2 ulps
        r = r0
        for _ in range(abs(k)):
            r = np.nextafter(r, F32(np.inf) if k > 0 else F32(-np.inf)).astype(F32)
        a = (d * r).astype(F32)
        assert float(a.max()) < 31.0
        near = np.abs(a - np.floor(a) - F32(0.5)) <= F32(4e-5)
        bad += int(np.sum((np.rint(a) != np.rint(q)) & ~near))
    return bad


def test_reciprocal_quotient_rounds_like_the_division():
    rng = np.random.default_rng(0)
    for scale in (0.02, 1.0, 1e-3, 1e-5, 3e-7, 100.0):   # 3e-7: subnormal f16 scales
        w = (rng.standard_normal((20000, 64)) * scale).astype(np.float16).astype(F32)
        lo, hi = w.min(1), w.max(1)
        s = ((hi - lo).astype(F32) / F32(15)).astype(F32).astype(np.float16).astype(F32)
        ok = s != 0
        d = (w - lo[:, None]).astype(F32)
        assert _shortcut_mismatches(d[ok].ravel(), np.broadcast_to(s[:, None], w.shape)[ok].ravel()) == 0


def test_reciprocal_quotient_at_half_integers():
    rng = np.random.default_rng(1)
    s = np.concatenate([rng.uniform(1e-4, 1.0, 4000),
                        rng.integers(1, 1024, 4000) * 2.0 ** -24]).astype(np.float16).astype(F32)
    s = s[s > 0]
    for h in np.arange(0.5, 15.0, 1.0):
        for ulps in range(-4, 5):
            q = np.full(s.shape, F32(h))
            for _ in range(abs(ulps)):
                q = np.nextafter(q, F32(np.inf) if ulps > 0 else F32(-np.inf)).astype(F32)
            assert _shortcut_mismatches((q * s).astype(F32), s) == 0
