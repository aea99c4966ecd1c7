"""Host check of the level rule the gfx950 quantizer uses (no GPU needed).

The kernel takes a weight's level from t = fl(w * fl(1/s)) and falls back to
the IEEE quotient fl(w / s) only when t lies within 4e-6 of a half-integer.
That is bit-identical to rounding fl(w / s) for every weight as long as
|t - fl(w / s)| stays below 4e-6 whenever |w / s| <= 10.5 (the largest ratio a
binary16 scale max|w|/7 allows).  Here the same IEEE fp32 operations are
replayed in numpy over every finite positive binary16 scale, with weights at
and around every midpoint (h + 1/2) * s, and the two routes are compared.
"""
import numpy as np


def _fast_levels(w, s):
    r = np.float32(1.0) / s
    t = (w * r).astype(np.float32)
    n = np.rint(t)
    near = np.abs(t - n) >= np.float32(0.5) - np.float32(4e-6)
    exact = np.rint((w / s).astype(np.float32))
    return np.clip(np.where(near, exact, n), -8, 7), near


def test_fast_level_rule_matches_ieee_quotient_for_every_scale():
    bits = np.arange(1, 0x7C00, dtype=np.uint16)                 # every finite positive fp16
    s = bits.view(np.float16).astype(np.float32)
    halves = np.arange(-11, 11, dtype=np.float64) + 0.5          # |w / s| up to 10.5
    steps = np.arange(-4, 5)
    checked = fell_back = 0
    for h in halves:
        w0 = (np.float64(h) * s.astype(np.float64)).astype(np.float32)
        for k in steps:
            w = w0.copy()
            if k > 0:
                for _ in range(k):
                    w = np.nextafter(w, np.float32(np.inf))
            elif k < 0:
                for _ in range(-k):
                    w = np.nextafter(w, np.float32(-np.inf))
            with np.errstate(over="ignore", invalid="ignore"):
                lv, near = _fast_levels(w, s)
                ref = np.clip(np.rint((w / s).astype(np.float32)), -8, 7)
            ok = np.isfinite(w)
            assert np.array_equal(lv[ok], ref[ok]), (h, k)
            checked += int(ok.sum())
            fell_back += int((near & ok).sum())
    assert checked > 1_000_000 and fell_back > 0


def test_fast_level_rule_on_spread_weights():
    rng = np.random.default_rng(5)
    for _ in range(20):
        w = (rng.standard_normal((4096, 32)) * 10.0 ** rng.uniform(-6, 3)).astype(np.float32)
        amax = np.abs(w).max(axis=1, keepdims=True)
        s = (amax / np.float32(7)).astype(np.float32).astype(np.float16).astype(np.float32)
        keep = (s != 0).ravel()
        w, s = w[keep], s[keep]
        lv, _ = _fast_levels(w, s)
        ref = np.clip(np.rint((w / s).astype(np.float32)), -8, 7)
        assert np.array_equal(lv, ref)
