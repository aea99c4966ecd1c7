"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each pin takes an ``oracle.Oracle`` (so that the same pins can be run against
deliberately broken copies of it) and raises AssertionError on a mismatch.

What pins what:
  golden_groups        hand-worked groups (tests/golden/q4_groups.txt): scale
                       rule, rounding ties, clamp, zero-scale rule, nibble order
  golden_product       the hand-worked product of group A with x = 1
  f16_conversion       the oracle's binary16 converter vs numpy's (an
                       independent round-to-nearest-even implementation)
  scale_vs_numpy       scale = numpy.float16(numpy.float32(max|w|) / 7)
  levels_brute_force   every level is the nearest of the 16 table levels to w
                       (ties to even), found by exhaustive search in fp64
  invariants           |w - s*q| <= s/2 for unclamped w; the group's largest
                       |w| gets |q| = 7 when s is normal; codes in 0..15
  product_vs_numpy     fp64 product vs numpy matmul on an independently
                       unpacked and dequantized W (several groups and rows)
  product_exact        exact rational product (fractions.Fraction) on small K
  product_special      x = 0, W = 0, one-hot x exposes every s*q exactly
  errors               shape, non-finite and overflow inputs are rejected
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "q4_groups.txt")


# --------------------------------------------------------------------------
# helpers independent of the oracle
# --------------------------------------------------------------------------

def load_golden(path: str = GOLDEN):
    groups = {}
    cur = None
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "group":
                cur = {}
                groups[rest.strip()] = cur
            elif key == "w":
                bits = np.array([int(t, 16) for t in rest.split()], dtype=np.uint32)
                cur["w"] = bits.view(np.float32)
            elif key == "scale":
                cur["scale"] = int(rest, 16)
            elif key == "q":
                cur["q"] = np.array([int(t) for t in rest.split()], dtype=np.int64)
            elif key == "bytes":
                cur["bytes"] = np.array([int(t, 16) for t in rest.split()], dtype=np.uint8)
            elif key == "product_x_ones":
                y, b = rest.split()
                cur["product"] = (float(y), float(b))
    return groups


def unpack_levels(packed: np.ndarray) -> np.ndarray:
    """uint8 [n, k/2] -> int levels [n, k]: low nibble = even element."""
    lo = (packed & 0x0F).astype(np.int64) - 8
    hi = (packed >> 4).astype(np.int64) - 8
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.int64)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def dequantize_f64(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    q = unpack_levels(packed).astype(np.float64)
    s = scales.view(np.float16).astype(np.float64)
    return q * np.repeat(s, 32, axis=1)


def spread_weights(rng, n, k):
    """Groups whose magnitudes span tiny (subnormal-scale) to large."""
    w = rng.standard_normal((n, k)).astype(np.float32)
    mag = 10.0 ** rng.uniform(-9, 4, size=(n, k // 32, 1))
    w = (w.reshape(n, k // 32, 32) * mag).reshape(n, k).astype(np.float32)
    return w


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------

def golden_groups(o):
    for name, g in load_golden().items():
        packed, scales = o.quantize(g["w"].reshape(1, 32))
        assert int(scales[0, 0]) == g["scale"], (name, hex(int(scales[0, 0])))
        assert np.array_equal(packed[0], g["bytes"]), (name, packed[0])
        assert np.array_equal(unpack_levels(packed)[0], g["q"]), name


def golden_product(o):
    g = load_golden()["A"]
    packed, scales = o.quantize(g["w"].reshape(1, 32))
    y, bound = o.matmul(np.ones((1, 32), np.float16), packed, scales)
    assert (y[0, 0], bound[0, 0]) == g["product"], (y, bound)


def _f16_edge_values():
    v = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6,
         2.0 ** -14, 2.0 ** -24, 2.0 ** -25, 1.5 * 2.0 ** -25, 2.0 ** -26,
         3 * 2.0 ** -25, 5 * 2.0 ** -25, 1023.5 * 2.0 ** -24, 1024.5 * 2.0 ** -24,
         1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2048.0 + 1.0, 2048.0 + 3.0,
         np.float32(1.4e-45), np.inf, -np.inf]
    for e in range(-26, 16):            # exact ties in every binade
        for frac in (0.5, 1.5, 2.5, 1023.5):
            v.append((1024 + frac) * 2.0 ** (e - 10))
    return np.array(v, dtype=np.float32)


def f16_conversion(o):
    rng = np.random.default_rng(1234)
    vals = np.concatenate([
        _f16_edge_values(),
        (rng.standard_normal(4000) * 10.0 ** rng.uniform(-9, 5, 4000)).astype(np.float32),
        rng.integers(0, 2 ** 32, 4000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    vals = vals[~np.isnan(vals)]
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([o.f32_to_f16_bits(float(v)) for v in vals], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(vals[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]
    # widening is exact: compare with numpy's binary16 -> float64
    allbits = np.arange(0, 65536, 97, dtype=np.uint16)
    allbits = allbits[(allbits & 0x7C00) != 0x7C00]
    back = np.array([o.f16_bits_to_f64(int(h)) for h in allbits])
    assert np.array_equal(back, allbits.view(np.float16).astype(np.float64))


def scale_vs_numpy(o):
    rng = np.random.default_rng(7)
    w = spread_weights(rng, 64, 32 * 40)
    _, scales = o.quantize(w)
    amax = np.abs(w.reshape(64, 40, 32)).max(axis=2).astype(np.float32)
    ref = (amax / np.float32(7.0)).astype(np.float32).astype(np.float16).view(np.uint16)
    assert np.array_equal(scales, ref)
    # no double rounding: the exact quotient rounds to the same binary16
    ref64 = (amax.astype(np.float64) / 7.0).astype(np.float16).view(np.uint16)
    assert np.array_equal(scales, ref64)


def _tie_groups(rng, n_groups):
    """Groups whose scale is known in advance (the first element is 7*s, so
    max|w|/7 == s exactly) and whose other elements sit exactly on the
    midpoints (h + 1/2)*s between two levels, or one fp32 ulp either side."""
    out = np.empty((n_groups, 32), dtype=np.float32)
    halves = np.arange(-6.5, 7.0, 1.0)
    for g in range(n_groups):
        if g % 4 == 0:
            s = np.float16(int(rng.integers(1, 1024)) * 2.0 ** -24)   # subnormal scale
        else:
            s = np.float16(10.0 ** rng.uniform(-4, 3))
        s32 = np.float32(s)
        vals = (rng.choice(halves, 31) * np.float64(s32)).astype(np.float32)
        nudge = rng.integers(-1, 2, 31)
        vals = np.where(nudge > 0, np.nextafter(vals, np.float32(np.inf)), vals)
        vals = np.where(nudge < 0, np.nextafter(vals, np.float32(-np.inf)), vals)
        out[g, 0] = np.float32(7) * s32
        out[g, 1:] = vals
    return out


def levels_brute_force(o):
    rng = np.random.default_rng(11)
    w = np.concatenate([spread_weights(rng, 32, 32 * 24),
                        _tie_groups(rng, 32 * 24).reshape(32, 32 * 24)])
    packed, scales = o.quantize(w)
    s = scales.view(np.float16).astype(np.float64)
    sg = np.repeat(s, 32, axis=1)
    q = unpack_levels(packed)
    levels = np.arange(-8, 8, dtype=np.float64)
    dist = np.abs(w.astype(np.float64)[..., None] - sg[..., None] * levels)  # exact in fp64
    is_best = dist == dist.min(axis=-1, keepdims=True)
    even = (np.arange(-8, 8) % 2 == 0)
    pick_even = is_best & even
    choice = np.where(pick_even.any(-1), np.argmax(pick_even, -1), np.argmax(is_best, -1))
    ref = levels[choice].astype(np.int64)
    ref[sg == 0] = 0
    bad = np.nonzero(q != ref)
    assert bad[0].size == 0, [(float(w[i, j]), float(sg[i, j]), int(q[i, j]), int(ref[i, j]))
                              for i, j in zip(*bad)][:5]
    # the planted groups really carry their planned scale and real ties
    planted = w[32:].reshape(-1, 32)
    assert np.array_equal(scales[32:].reshape(-1).view(np.float16).astype(np.float32) * 7,
                          planted[:, 0])
    assert np.any(is_best.sum(-1) > 1)


def invariants(o):
    rng = np.random.default_rng(5)
    w = spread_weights(rng, 40, 32 * 16)
    packed, scales = o.quantize(w)
    s = np.repeat(scales.view(np.float16).astype(np.float64), 32, axis=1)
    q = unpack_levels(packed)
    assert q.min() >= -8 and q.max() <= 7
    wd = w.astype(np.float64)
    unclamped = (s > 0) & (wd <= 7.5 * s) & (wd >= -8.5 * s)
    err = np.abs(wd - s * q)
    assert np.all(err[unclamped] <= s[unclamped] / 2)
    # argmax element reaches |q| = 7 when the scale is a normal binary16
    normal = (scales & 0x7C00) != 0
    amax_idx = np.abs(w.reshape(40, 16, 32)).argmax(axis=2)
    qa = np.take_along_axis(q.reshape(40, 16, 32), amax_idx[..., None], 2)[..., 0]
    assert np.all(np.abs(qa[normal]) == 7)


def product_vs_numpy(o):
    rng = np.random.default_rng(3)
    for (m, n, k) in [(1, 7, 96), (3, 5, 256), (8, 33, 128)]:
        w = spread_weights(rng, n, k)
        x = (rng.standard_normal((m, k)) * 3).astype(np.float16)
        packed, scales = o.quantize(w)
        y, bound = o.matmul(x, packed, scales)
        wd = dequantize_f64(packed, scales)
        xd = x.astype(np.float64)
        ref = xd @ wd.T
        ref_bound = np.abs(xd) @ np.abs(wd).T
        assert np.all(np.abs(y - ref) <= 1e-12 * ref_bound + 1e-300)
        assert np.allclose(bound, ref_bound, rtol=1e-12, atol=0)


def product_exact(o):
    rng = np.random.default_rng(9)
    for (m, n, k) in [(1, 1, 32), (2, 2, 64)]:
        w = (rng.standard_normal((n, k)) * 0.05).astype(np.float32)
        x = rng.standard_normal((m, k)).astype(np.float16)
        packed, scales = o.quantize(w)
        y, bound = o.matmul(x, packed, scales)
        q = unpack_levels(packed)
        for i in range(m):
            for r in range(n):
                tot = Fraction(0)
                tot_abs = Fraction(0)
                for j in range(k // 32):
                    s = Fraction(float(scales.view(np.float16)[r, j]))
                    for t in range(32):
                        xv = Fraction(float(x[i, 32 * j + t]))
                        tot += s * xv * int(q[r, 32 * j + t])
                        tot_abs += abs(s * xv * int(q[r, 32 * j + t]))
                assert abs(Fraction(float(y[i, r])) - tot) <= tot_abs * Fraction(1, 2 ** 50)
                assert abs(Fraction(float(bound[i, r])) - tot_abs) <= tot_abs * Fraction(1, 2 ** 50)


def product_special(o):
    rng = np.random.default_rng(21)
    n, k = 3, 64
    w = (rng.standard_normal((n, k)) * 0.3).astype(np.float32)
    packed, scales = o.quantize(w)
    y, b = o.matmul(np.zeros((2, k), np.float16), packed, scales)
    assert np.all(y == 0) and np.all(b == 0)
    zp, zs = o.quantize(np.zeros((n, k), np.float32))
    y, _ = o.matmul(rng.standard_normal((2, k)).astype(np.float16), zp, zs)
    assert np.all(y == 0)
    onehot = np.eye(k, dtype=np.float16)                 # row e selects element e
    y, _ = o.matmul(onehot, packed, scales)
    q = unpack_levels(packed)
    s = np.repeat(scales.view(np.float16).astype(np.float64), 32, axis=1)
    assert np.array_equal(y, (s * q).T)


def errors(o):
    st, _, _ = o.quantize_status(np.zeros((2, 48), np.float32))
    assert st == 2
    w = np.zeros((2, 64), np.float32)
    w[1, 5] = np.nan
    assert o.quantize_status(w)[0] == 3
    w[1, 5] = np.inf
    assert o.quantize_status(w)[0] == 3
    w[1, 5] = 7 * 65520.0
    assert o.quantize_status(w)[0] == 3
    w[1, 5] = 7 * 65504.0                                 # largest finite scale
    st, _, sc = o.quantize_status(w)
    assert st == 0 and int(sc[1, 0]) == 0x7BFF


# -- the product with fp16 weights -------------------------------------------

def f16_product_vs_numpy(o):
    rng = np.random.default_rng(31)
    for (m, n, k) in [(1, 7, 96), (3, 5, 40), (8, 33, 128)]:
        x = (rng.standard_normal((m, k)) * 3).astype(np.float16)
        w = (rng.standard_normal((n, k)) * 0.05).astype(np.float16)
        y, bound = o.matmul_f16(x, w)
        xd, wd = x.astype(np.float64), w.astype(np.float64)
        ref = xd @ wd.T
        ref_bound = np.abs(xd) @ np.abs(wd).T
        assert np.all(np.abs(y - ref) <= 1e-12 * ref_bound + 1e-300)
        assert np.allclose(bound, ref_bound, rtol=1e-12, atol=0)


def f16_product_exact(o):
    rng = np.random.default_rng(33)
    m, n, k = 2, 3, 24
    x = rng.standard_normal((m, k)).astype(np.float16)
    w = (rng.standard_normal((n, k)) * 0.1).astype(np.float16)
    y, bound = o.matmul_f16(x, w)
    for i in range(m):
        for r in range(n):
            terms = [Fraction(float(x[i, t])) * Fraction(float(w[r, t])) for t in range(k)]
            tot, tot_abs = sum(terms), sum(abs(t) for t in terms)
            assert abs(Fraction(float(y[i, r])) - tot) <= tot_abs * Fraction(1, 2 ** 50)
            assert abs(Fraction(float(bound[i, r])) - tot_abs) <= tot_abs * Fraction(1, 2 ** 50)


def f16_product_special(o):
    rng = np.random.default_rng(35)
    n, k = 4, 40
    w = rng.standard_normal((n, k)).astype(np.float16)
    y, _ = o.matmul_f16(np.eye(k, dtype=np.float16), w)      # row e selects element e
    assert np.array_equal(y, w.astype(np.float64).T)
    y, b = o.matmul_f16(np.zeros((2, k), np.float16), w)
    assert np.all(y == 0) and np.all(b == 0)
    y, _ = o.matmul_f16(rng.standard_normal((2, k)).astype(np.float16), np.zeros((n, k), np.float16))
    assert np.all(y == 0)
    xp = np.abs(rng.standard_normal((1, k))).astype(np.float16)
    y, b = o.matmul_f16(xp, np.abs(w))                        # all terms >= 0: bound == y
    assert np.array_equal(y, b)
    y, b = o.matmul_f16(xp, -np.abs(w))                       # all terms <= 0: bound == -y
    assert np.array_equal(-y, b)


def f16_errors(o):
    st = o.lib.q4o_matmul_f16(None, None, 1, 1, 32, None, None)
    assert st == 1
    x = np.zeros((1, 8), np.uint16)
    out = np.zeros((1, 1))
    assert o.lib.q4o_matmul_f16(x.ctypes.data, x.ctypes.data, 1, 1, 0, out.ctypes.data, None) == 2


ALL_PINS = [golden_groups, golden_product, f16_conversion, scale_vs_numpy,
            levels_brute_force, invariants, product_vs_numpy, product_exact,
            product_special, errors, f16_product_vs_numpy, f16_product_exact,
            f16_product_special, f16_errors]
