"""GPU parity: the gfx950 library (through its C ABI) against the CPU oracle.

Bars:
  q4_quantize        bit-exact packed codes and fp16 scales
  q4_gemv / q4_gemm  |y - y_ref| <= 1e-3 * sum|x*s*q| + 1e-6 for every output,
                     exact where the result is exactly representable (one-hot x,
                     x = 0, W = 0)
Small cases span several tiles plus ragged tails and are compared in full;
the five workload configurations run at full size and are compared on
sampled rows (all m) that the oracle recomputes one by one.
"""
import sys

import numpy as np
import pytest

import oracle
import oracle_pins
import q4_inputs as qi

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _log(msg):
    print("[parity] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def q4():
    import q4_group_quantized_amd as mod
    assert torch.cuda.is_available(), "GPU tests need a device"
    mod.load()
    return mod


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


DEV = "cuda:0"


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def gpu_quantize(q4, w):
    packed, scales = q4.q4_quantize(gpu(w))
    torch.cuda.synchronize()
    return packed.cpu().numpy(), scales.cpu().numpy().view(np.uint16)


def product(q4, fn, x, packed, scales):
    y = getattr(q4, fn)(gpu(x), gpu(packed), gpu(scales.view(np.float16)))
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def assert_within(y, y_ref, bound, what):
    err = np.abs(y - y_ref)
    tol = oracle.tolerance(bound)
    bad = np.argwhere(~(err <= tol))
    assert bad.size == 0, "%s: %d outputs outside tolerance, first %s: y=%r ref=%r tol=%r" % (
        what, len(bad), tuple(bad[0]), y[tuple(bad[0])], y_ref[tuple(bad[0])], tol[tuple(bad[0])])


# --------------------------------------------------------------------------
# quantizer
# --------------------------------------------------------------------------

def test_quantize_golden_groups(q4, orc):
    golden = oracle_pins.load_golden()
    w = np.stack([g["w"] for g in golden.values()])           # one group per row
    _log("quantize golden groups %s" % (w.shape,))
    packed, scales = gpu_quantize(q4, w)
    for i, g in enumerate(golden.values()):
        assert int(scales[i, 0]) == g["scale"]
        assert np.array_equal(packed[i], g["bytes"])
    wrow = w.reshape(1, -1)                                    # the same groups in one row
    packed, scales = gpu_quantize(q4, wrow)
    rp, rs = orc.quantize(wrow)
    assert np.array_equal(packed, rp) and np.array_equal(scales, rs)


@pytest.mark.parametrize("n,k", [(1, 32), (3, 96), (17, 160), (64, 2560), (1000, 1024),
                                 (33, 32 * 37), (5, 65536), (2, 2 ** 24)])
def test_quantize_bit_exact(q4, orc, n, k):
    rng = np.random.default_rng(n * 7919 + k)
    w = oracle_pins.spread_weights(rng, n, k)
    if k >= 64:
        w[0, :32 * min(8, k // 32)] = oracle_pins._tie_groups(rng, min(8, k // 32)).reshape(-1)
    w[-1, :32] = 0.0
    _log("quantize n=%d k=%d" % (n, k))
    packed, scales = gpu_quantize(q4, w)
    rp, rs = orc.quantize(w)
    assert np.array_equal(scales, rs), np.argwhere(scales != rs)[:5]
    assert np.array_equal(packed, rp), np.argwhere(packed != rp)[:5]


def test_quantize_midpoints_everywhere(q4, orc):
    """Every group a tie group (weights on level midpoints and one ulp either
    side, normal and subnormal scales): the kernel's midpoint fallback runs in
    many lanes of many waves at once."""
    rng = np.random.default_rng(2024)
    n, k = 256, 1024
    w = oracle_pins._tie_groups(rng, n * k // 32).reshape(n, k)
    _log("quantize midpoints n=%d k=%d" % (n, k))
    packed, scales = gpu_quantize(q4, w)
    rp, rs = orc.quantize(w)
    assert np.array_equal(scales, rs), np.argwhere(scales != rs)[:5]
    assert np.array_equal(packed, rp), np.argwhere(packed != rp)[:5]


# --------------------------------------------------------------------------
# products on small shapes, compared in full
# --------------------------------------------------------------------------

# at m = 2..8 the first seven take the GEMM's small-batch tiles (n <= 4096 rows),
# the last two the block-diagonal GEMV (ragged row blocks, partial last step)
SHAPES = [(1, 32), (15, 64), (17, 96), (33, 256), (100, 1056), (257, 2560), (1024, 1024),
          (4097, 96), (4110, 2560)]


def _case(orc, m, n, k, seed):
    rng = np.random.default_rng(seed)
    w = oracle_pins.spread_weights(rng, n, k) if seed % 2 else \
        (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = (rng.standard_normal((m, k)) * 2).astype(np.float16)
    packed, scales = orc.quantize(w)
    y_ref, bound = orc.matmul(x, packed, scales)
    return x, packed, scales, y_ref, bound


@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("fn", ["q4_gemv", "q4_gemm"])
def test_decode_product(q4, orc, fn, m, n, k):
    x, packed, scales, y_ref, bound = _case(orc, m, n, k, seed=m * 1000 + n + k)
    _log("%s m=%d n=%d k=%d" % (fn, m, n, k))
    y = product(q4, fn, x, packed, scales)
    assert_within(y, y_ref, bound, "%s m=%d n=%d k=%d" % (fn, m, n, k))


@pytest.mark.parametrize("k", [256, 512, 768, 1024, 1280, 1536, 1792, 2048, 2304, 2560, 3072,
                               3584, 4096, 5120, 6144, 8192])
@pytest.mark.parametrize("n", [1, 3, 5, 61, 4099])
def test_single_token_streaming(q4, orc, n, k):
    """m = 1 streaming kernel: every lanes-per-row / groups-per-lane variant,
    ragged row counts (not a multiple of the rows per wave step)."""
    x, packed, scales, y_ref, bound = _case(orc, 1, n, k, seed=n * 13 + k)
    _log("q4_gemv m=1 n=%d k=%d" % (n, k))
    y = product(q4, "q4_gemv", x, packed, scales)
    assert_within(y, y_ref, bound, "q4_gemv m=1 n=%d k=%d" % (n, k))


@pytest.mark.parametrize("m", [9, 15, 16, 17, 24, 31, 32, 33, 64, 100, 128, 129, 300, 1024,
                               1100])
@pytest.mark.parametrize("n,k", [(17, 96), (64, 256), (130, 2560), (200, 160), (70, 1056)])
def test_prefill_product(q4, orc, m, n, k):
    x, packed, scales, y_ref, bound = _case(orc, m, n, k, seed=m * 31 + n * 7 + k)
    _log("q4_gemm m=%d n=%d k=%d" % (m, n, k))
    y = product(q4, "q4_gemm", x, packed, scales)
    assert_within(y, y_ref, bound, "q4_gemm m=%d n=%d k=%d" % (m, n, k))


TILING_CASES = [(64, 1000, 256), (256, 4096, 256), (384, 4096, 128), (512, 4096, 256),
                (520, 4100, 160), (1024, 4096, 256), (600, 4098, 96), (1030, 4100, 96)]


@pytest.mark.parametrize("m,n,k", TILING_CASES, ids=["m%d-n%d-k%d" % c for c in TILING_CASES])
def test_prefill_every_tile_shape(q4, orc, m, n, k):
    """Shapes for which the GEMM picks each of its tile shapes on a 256-CU
    device, compared in full: 32x64 (16-group stages, here one partial stage)
    and 64x64; 64x128 with a group count that is and is not a multiple of its
    8-group stage; 128x128 with and without a partial last stage, with ragged
    rows and columns, and with n % 4 != 0 (element-wise stores)."""
    x, packed, scales, y_ref, bound = _case(orc, m, n, k, seed=m + n + k)
    _log("q4_gemm m=%d n=%d k=%d" % (m, n, k))
    y = product(q4, "q4_gemm", x, packed, scales)
    assert_within(y, y_ref, bound, "q4_gemm m=%d n=%d k=%d" % (m, n, k))


@pytest.mark.parametrize("m,k", [(4, 15360), (4, 15392), (8, 7680), (8, 7712), (5, 1504),
                                 (2, 4160)])
@pytest.mark.parametrize("n", [5, 4099])
def test_blockdiag_lds_limits(q4, orc, m, n, k):
    """m = 2..8 at the largest k whose activations and step buffers fit in LDS
    (15360 for m <= 4, 7680 for m = 5..8) and just past it (chunked kernel),
    and k whose group count is not a multiple of the 16 groups of a step."""
    x, packed, scales, y_ref, bound = _case(orc, m, n, k, seed=m * 7 + n + k)
    _log("q4_gemv m=%d n=%d k=%d" % (m, n, k))
    y = product(q4, "q4_gemv", x, packed, scales)
    assert_within(y, y_ref, bound, "q4_gemv m=%d n=%d k=%d" % (m, n, k))


SCALE_OFFSET_CASES = [("q4_gemv", 1, 1024, 37), ("q4_gemv", 2, 1024, 37),
                      ("q4_gemv", 5, 544, 37), ("q4_gemv", 8, 7936, 37),
                      ("q4_gemv", 3, 16384, 37), ("q4_gemv", 2, 1024, 4099),
                      ("q4_gemv", 8, 2560, 4099), ("q4_gemv", 5, 544, 4099),
                      ("q4_gemm", 40, 1024, 37),
                      ("q4_gemm", 16, 1056, 37), ("q4_gemm", 32, 1056, 37),
                      ("q4_gemm", 512, 256, 4096), ("q4_gemm", 1024, 256, 4096)]


@pytest.mark.parametrize("fn,m,k,n", SCALE_OFFSET_CASES,
                         ids=["%s-m%d-k%d-n%d" % c for c in SCALE_OFFSET_CASES])
@pytest.mark.parametrize("offset", [1, 2, 4, 8])
def test_scales_at_any_even_address(q4, orc, fn, m, k, n, offset):
    """The scale matrix need only be 2-byte aligned: it is placed `offset`
    fp16 elements past a 256-byte boundary (2, 4, 8 and 16 bytes), so the
    kernels whose wide scale loads need 4, 8 or 16 bytes (m = 2..8 with a
    whole number of steps or tiles; the 64x128 and 128x128 GEMM tiles) must
    take their 2-byte form there.  Every offset gives the bits of the
    aligned call."""
    x, packed, scales, y_ref, bound = _case(orc, m, n, k, seed=m + k + offset)
    _log("%s m=%d n=%d k=%d scales at +%d B" % (fn, m, n, k, 2 * offset))
    y0 = product(q4, fn, x, packed, scales)
    buf = torch.zeros(scales.size + 16, dtype=torch.float16, device=DEV)
    shifted = buf[offset:offset + scales.size].view(scales.shape)
    shifted.copy_(gpu(scales.view(np.float16)))
    assert shifted.data_ptr() % 256 == 2 * offset
    y = getattr(q4, fn)(gpu(x), gpu(packed), shifted)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    assert np.array_equal(y.view(np.uint32), y0.astype(np.float32).view(np.uint32))
    assert_within(y.astype(np.float64), y_ref, bound, "%s scales at +%d B" % (fn, 2 * offset))


@pytest.fixture(scope="module")
def max_rows_matrix():
    """n = 2^31 - 1 rows (the largest n the contract allows) at k = 32: random
    codes and scales in [0.001, 0.01] generated on the device (38 GB)."""
    n, k = 2 ** 31 - 1, 32
    g = torch.Generator(device=DEV)
    g.manual_seed(2 ** 31 - 1)
    packed = torch.empty((n, k // 2), dtype=torch.uint8, device=DEV).random_(0, 256, generator=g)
    scales = torch.empty((n, 1), dtype=torch.float16, device=DEV).uniform_(0.001, 0.01,
                                                                            generator=g)
    torch.cuda.synchronize()
    yield packed, scales
    del packed, scales
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fn,m", [("q4_gemv", 1), ("q4_gemv", 2), ("q4_gemm", 9)])
def test_maximum_rows(q4, orc, max_rows_matrix, fn, m):
    """Row offsets past 2^32 bytes, and for q4_gemm 67 million tiles: more than
    one launch's grid holds, so the tiles are spread over several launches.
    Sampled rows -- the ends, launch-chunk and power-of-two boundaries, and
    random ones -- are recomputed by the oracle."""
    packed, scales = max_rows_matrix
    n, k = packed.shape[0], packed.shape[1] * 2
    rng = np.random.default_rng(m)
    x = (rng.standard_normal((m, k)) * 2).astype(np.float16)
    _log("%s m=%d n=%d k=%d" % (fn, m, n, k))
    y = getattr(q4, fn)(gpu(x), packed, scales)
    torch.cuda.synchronize()
    rows = {0, 1, 31, 32, 2 ** 25 - 1, 2 ** 25, 2 ** 25 + 32, 2 ** 27 + 5, 2 ** 28 - 1, 2 ** 28,
            2 ** 31 - 2 ** 20, n - 33, n - 2, n - 1}
    rows |= set(int(r) for r in rng.integers(0, n, 64))
    rows = np.array(sorted(rows))
    idx = torch.from_numpy(rows).to(DEV)
    rp = packed[idx].cpu().numpy()
    rs = scales[idx].cpu().numpy().view(np.uint16)
    y_rows = y[:, idx].cpu().numpy().astype(np.float64)
    del y
    torch.cuda.empty_cache()
    y_ref, bound = orc.matmul(x, rp, rs)
    assert_within(y_rows, y_ref, bound, "%s m=%d at n = 2^31 - 1" % (fn, m))


@pytest.mark.parametrize("fn,m,k", [("q4_gemv", 1, 65536), ("q4_gemv", 8, 65536),
                                    ("q4_gemm", 40, 65536), ("q4_gemm", 16, 65536),
                                    ("q4_gemm", 32, 65536), ("q4_gemv", 1, 2 ** 20),
                                    ("q4_gemv", 1, 2 ** 24), ("q4_gemv", 8, 2 ** 24),
                                    ("q4_gemm", 9, 2 ** 24)])
def test_long_k(q4, orc, fn, m, k):
    """K beyond what one LDS pass of activations holds, up to the largest k
    the contract allows (2^24)."""
    x, packed, scales, y_ref, bound = _case(orc, m, 3, k, seed=k + m)
    _log("%s m=%d n=3 k=%d" % (fn, m, k))
    y = product(q4, fn, x, packed, scales)
    assert_within(y, y_ref, bound, "%s long k" % fn)


@pytest.mark.parametrize("fn", ["q4_gemv", "q4_gemm"])
def test_exact_special_inputs(q4, orc, fn):
    rng = np.random.default_rng(77)
    n, k = 37, 96
    w = oracle_pins.spread_weights(rng, n, k)
    packed, scales = orc.quantize(w)
    q = oracle_pins.unpack_levels(packed).astype(np.float64)
    s = np.repeat(scales.view(np.float16).astype(np.float64), 32, axis=1)
    _log("%s one-hot / zero inputs" % fn)
    step = 8 if fn == "q4_gemv" else k
    for e0 in range(0, k, step):
        x = np.eye(k, dtype=np.float16)[e0:e0 + step]
        y = product(q4, fn, x, packed, scales)
        assert np.array_equal(y, (s * q).T[e0:e0 + step]), "one-hot rows %d.." % e0
    y = product(q4, fn, np.zeros((3, k), np.float16), packed, scales)
    assert np.all(y == 0)
    zp, zs = orc.quantize(np.zeros((n, k), np.float32))
    y = product(q4, fn, rng.standard_normal((3, k)).astype(np.float16), zp, zs)
    assert np.all(y == 0)


@pytest.mark.parametrize("fn,m", [("q4_gemv", 1), ("q4_gemv", 8), ("q4_gemm", 200)])
def test_deterministic(q4, orc, fn, m):
    x, packed, scales, _, _ = _case(orc, m, 999, 2560, seed=5)
    _log("%s determinism m=%d" % (fn, m))
    a = product(q4, fn, x, packed, scales)
    b = product(q4, fn, x, packed, scales)
    assert np.array_equal(a, b)


def test_non_default_stream(q4, orc):
    x, packed, scales, y_ref, bound = _case(orc, 4, 300, 1024, seed=3)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        xg, pg, sg = gpu(x), gpu(packed), gpu(scales.view(np.float16))
        y = q4.q4_gemv(xg, pg, sg)
    s.synchronize()
    assert_within(y.cpu().numpy().astype(np.float64), y_ref, bound, "stream")


def test_binding_rejects_bad_calls(q4):
    x = torch.zeros((9, 64), dtype=torch.float16, device=DEV)
    p = torch.zeros((4, 32), dtype=torch.uint8, device=DEV)
    s = torch.zeros((4, 2), dtype=torch.float16, device=DEV)
    with pytest.raises(q4.Q4Error):
        q4.q4_gemv(x, p, s)
    with pytest.raises(ValueError):
        q4.q4_gemm(x, p[:, :16], s)


# --------------------------------------------------------------------------
# several matrices over one x in one call (q4_gemv_multi)
# --------------------------------------------------------------------------

MULTI_SETS = [
    (1, 1024, (1, 17, 300, 4099)),
    (1, 2560, (61, 5, 1000, 3, 257, 64, 9, 2)),      # eight matrices, ragged rows
    (1, 512, (1,)),
    (1, 8192, (5, 61)),
    (1, 96, (17, 33)),                               # k outside the streaming kernel
    (2, 256, (15, 100)),
    (8, 1056, (33, 7, 64)),
    (4, 2560, (61, 5, 1000, 3, 257, 64, 9, 2)),      # m <= 4 tile, eight matrices
    (5, 1024, (1, 17, 300, 4099)),
    (8, 2560, (2048, 2048, 4096)),                   # 4B DeltaNet q/k/v rows
    (7, 96, (17, 33)),                               # G = 3: partial step
    (8, 8192, (5, 61, 700)),                         # activations too large: chunked
    (3, 16384, (40, 3)),
    (8, 2560, (4096, 4097, 1, 5000)),                # both sides of the GEMV/tile split
    (2, 1024, (4100, 8, 4096)),
]


@pytest.mark.parametrize("m,k,ns", MULTI_SETS, ids=["m%d-k%d-%dmat" % (c[0], c[1], len(c[2]))
                                                    for c in MULTI_SETS])
def test_gemv_multi(q4, orc, m, k, ns):
    """Each output against the oracle, and bit-identical to q4_gemv alone."""
    rng = np.random.default_rng(m * 7 + k + len(ns))
    x = (rng.standard_normal((m, k)) * 2).astype(np.float16)
    mats, refs = [], []
    for i, n in enumerate(ns):
        w = oracle_pins.spread_weights(rng, n, k) if i % 2 else \
            (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
        packed, scales = orc.quantize(w)
        mats.append((gpu(packed), gpu(scales.view(np.float16))))
        refs.append(orc.matmul(x, packed, scales))
    _log("q4_gemv_multi m=%d k=%d n=%s" % (m, k, ns))
    xg = gpu(x)
    ys = q4.q4_gemv_multi(xg, mats)
    torch.cuda.synchronize()
    for i, (y, (y_ref, bound)) in enumerate(zip(ys, refs)):
        assert_within(y.cpu().numpy().astype(np.float64), y_ref, bound,
                      "multi matrix %d (n=%d)" % (i, ns[i]))
        alone = q4.q4_gemv(xg, *mats[i])
        torch.cuda.synchronize()
        assert torch.equal(y, alone), "multi matrix %d differs from q4_gemv" % i


@pytest.mark.parametrize("m", [1, 3, 8])
def test_gemv_multi_mixed_scale_alignment(q4, orc, m):
    """One matrix of the set has its scales only 2-byte aligned, so the whole
    launch takes the 2-byte scale loads; every output keeps the bits of
    q4_gemv on that matrix alone (which takes the wide loads where it can)."""
    rng = np.random.default_rng(90 + m)
    k, ns = 1024, (100, 2048, 33)
    x = (rng.standard_normal((m, k)) * 2).astype(np.float16)
    xg = gpu(x)
    mats, refs = [], []
    for i, n in enumerate(ns):
        packed, scales = orc.quantize((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
        sg = gpu(scales.view(np.float16))
        if i == 1:
            buf = torch.zeros(sg.numel() + 16, dtype=torch.float16, device=DEV)
            sg = buf[1:1 + sg.numel()].view(sg.shape)
            sg.copy_(gpu(scales.view(np.float16)))
            assert sg.data_ptr() % 8 == 2
        mats.append((gpu(packed), sg))
        refs.append(orc.matmul(x, packed, scales))
    _log("q4_gemv_multi m=%d k=%d n=%s, scales of matrix 1 at +2 B" % (m, k, ns))
    ys = q4.q4_gemv_multi(xg, mats)
    torch.cuda.synchronize()
    for i, (y, (y_ref, bound)) in enumerate(zip(ys, refs)):
        assert_within(y.cpu().numpy().astype(np.float64), y_ref, bound, "matrix %d" % i)
        alone = q4.q4_gemv(xg, mats[i][0], mats[i][1].clone())   # aligned copy
        torch.cuda.synchronize()
        assert torch.equal(y, alone), "multi matrix %d differs from q4_gemv" % i


def test_gemv_multi_binding_errors(q4):
    x = torch.zeros((1, 64), dtype=torch.float16, device=DEV)
    p = torch.zeros((4, 32), dtype=torch.uint8, device=DEV)
    s = torch.zeros((4, 2), dtype=torch.float16, device=DEV)
    with pytest.raises(q4.Q4Error):
        q4.q4_gemv_multi(x, [])
    with pytest.raises(q4.Q4Error):
        q4.q4_gemv_multi(x, [(p, s)] * 9)
    with pytest.raises(ValueError):
        q4.q4_gemv_multi(x, [(p, s), (p[:, :16], s[:, :1])])


GEMM_MULTI_SETS = [
    (9, 256, (15, 100)),
    (40, 1056, (33, 7, 64)),
    (16, 1056, (33, 7, 64)),                               # 16 x 16 tiles
    (24, 2560, (130, 5, 257)),                             # 32 x 16 tiles
    (32, 1056, (17, 100, 3, 64)),
    (128, 2560, (130, 5, 257, 64)),
    (300, 96, (17, 200, 3, 1, 70, 33, 9, 129)),            # eight matrices
    (512, 1024, (100, 61)),
    (1030, 256, (130, 61, 257)),                           # 64 x 64 tiles
    (512, 256, (2048, 1000, 777)),                         # 64 x 128 tiles (32x32 blocks)
    (1024, 160, (4096, 130, 3000)),                        # 128 x 128 tiles, partial stage
    (3, 256, (15, 100)),                                   # m <= 8: the q4_gemv_multi path
    (8, 1024, (4096, 4097, 17)),                           # m <= 8 on both sides of 4096 rows
]


@pytest.mark.parametrize("m,k,ns", GEMM_MULTI_SETS, ids=["m%d-k%d-%dmat" % (c[0], c[1], len(c[2]))
                                                         for c in GEMM_MULTI_SETS])
def test_gemm_multi(q4, orc, m, k, ns):
    """Each output against the oracle and the same bits on a second call; for
    m <= 32, where the tile shape follows m alone, bit-identical to q4_gemm on
    the matrix alone (above, the grouped launch may pick another tile shape
    and with it another order of the fp32 sums)."""
    rng = np.random.default_rng(m * 11 + k + len(ns))
    x = (rng.standard_normal((m, k)) * 2).astype(np.float16)
    mats, refs = [], []
    for i, n in enumerate(ns):
        w = oracle_pins.spread_weights(rng, n, k) if i % 2 else \
            (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
        packed, scales = orc.quantize(w)
        mats.append((gpu(packed), gpu(scales.view(np.float16))))
        refs.append(orc.matmul(x, packed, scales))
    _log("q4_gemm_multi m=%d k=%d n=%s" % (m, k, ns))
    xg = gpu(x)
    ys = q4.q4_gemm_multi(xg, mats)
    again = q4.q4_gemm_multi(xg, mats)
    torch.cuda.synchronize()
    for i, (y, (y_ref, bound)) in enumerate(zip(ys, refs)):
        assert_within(y.cpu().numpy().astype(np.float64), y_ref, bound,
                      "gemm multi matrix %d (n=%d)" % (i, ns[i]))
        assert torch.equal(y, again[i]), "gemm multi matrix %d not deterministic" % i
        alone = q4.q4_gemm(xg, *mats[i])
        torch.cuda.synchronize()
        assert_within(alone.cpu().numpy().astype(np.float64), y_ref, bound,
                      "q4_gemm matrix %d (n=%d)" % (i, ns[i]))
        if m <= 32:
            assert torch.equal(y, alone), "gemm multi matrix %d differs from q4_gemm" % i


def test_gemm_multi_layer_projections_full_size(q4, orc):
    """The six 4B projections of the decode set over one prefill batch (m = 512,
    outlier activations) in one launch: sampled rows against the oracle, for
    the grouped launch and for q4_gemm on each matrix alone."""
    wl = qi.WORKLOADS["decode_4b"]
    x = qi.activations(512, wl.cases[0][0].k, outliers=True)
    xg = gpu(x)
    mats, samples = [], []
    for mat, _ in wl.cases[:-1]:
        w = qi.weights(mat.n, mat.k, tensor_id=mat.tensor_id)
        mats.append(q4.q4_quantize(gpu(w)))
        rows = _sample_rows(mat.n, np.random.default_rng(mat.tensor_id), count=96)
        samples.append((rows, orc.quantize(w[rows])))
    _log("q4_gemm_multi: %d projections, m=512" % len(mats))
    ys = q4.q4_gemm_multi(xg, mats)
    torch.cuda.synchronize()
    for (mat, _), y, (p, s_), (rows, (rp, rs)) in zip(wl.cases, ys, mats, samples):
        alone = q4.q4_gemm(xg, p, s_)
        torch.cuda.synchronize()
        y_ref, bound = orc.matmul(x, rp, rs)
        assert_within(y.cpu().numpy().astype(np.float64)[:, rows], y_ref, bound, mat.name)
        assert_within(alone.cpu().numpy().astype(np.float64)[:, rows], y_ref, bound,
                      mat.name + " alone")


@pytest.mark.parametrize("key", ["decode_08b", "decode_4b"])
def test_gemv_multi_decode_set_full_size(q4, orc, key):
    """A whole decode set (seven matrices incl. the LM head) in one call, at
    full size: sampled rows against the oracle, every output bit-identical to
    q4_gemv on that matrix alone."""
    wl = qi.WORKLOADS[key]
    x = qi.activations(1, wl.cases[0][0].k, outliers=wl.outliers)
    xg = gpu(x)
    mats, samples = [], []
    for mat, _ in wl.cases:
        _log("%s %s: generating" % (key, mat.name))
        w = qi.weights(mat.n, mat.k, tensor_id=mat.tensor_id, wide_groups=mat.wide_groups)
        wg = gpu(w)
        mats.append(q4.q4_quantize(wg))
        del wg
        rows = _sample_rows(mat.n, np.random.default_rng(mat.tensor_id), count=128)
        samples.append((rows, orc.quantize(w[rows])))
        del w
    _log("%s: q4_gemv_multi over %d matrices" % (key, len(mats)))
    ys = q4.q4_gemv_multi(xg, mats)
    torch.cuda.synchronize()
    for (mat, _), y, (p, s), (rows, (rp, rs)) in zip(wl.cases, ys, mats, samples):
        assert torch.equal(y, q4.q4_gemv(xg, p, s)), mat.name
        y_ref, bound = orc.matmul(x, rp, rs)
        gy = y.cpu().numpy().astype(np.float64)[:, rows]
        assert_within(gy, y_ref, bound, "%s %s" % (key, mat.name))


# --------------------------------------------------------------------------
# LM-head top-k epilogue (q4_gemv_topk)
# --------------------------------------------------------------------------

def select_topk(y_row, topk):
    """The topk entries of one row of logits in the order the epilogue defines:
    value descending (+0 above -0, NaN last), then row ascending."""
    v = y_row.astype(np.float32)
    order = np.lexsort((np.arange(len(v)), np.signbit(v), -v.astype(np.float64)))
    return order[:topk]


def assert_valid_topk(sel, y_ref, bound, what):
    """`sel` (rows, best first) is a correct top-k of the oracle's products
    given that every logit may sit anywhere within its tolerance: for every
    selected row s and every row u ranked after it (later in the list, or not
    selected), y_ref[s] + tol[s] >= y_ref[u] - tol[u].  Several selections can
    pass when logits are closer than their tolerances; any of them is a
    correct greedy / top-k candidate set."""
    n = len(y_ref)
    sel = np.asarray(sel, dtype=np.int64)
    assert len(set(sel.tolist())) == len(sel), "%s: repeated rows %s" % (what, sel)
    assert np.all((sel >= 0) & (sel < n)), "%s: rows out of range" % what
    tol = oracle.tolerance(bound)
    hi = y_ref + tol
    lo = y_ref - tol
    rest = np.ones(n, dtype=bool)
    rest[sel] = False
    if rest.any():
        worst_sel = hi[sel].min()
        best_rest = lo[rest].max()
        assert worst_sel >= best_rest, (
            "%s: selected row %d (ref %.9g + tol) ranks below unselected row %d (ref %.9g - tol)"
            % (what, sel[np.argmin(hi[sel])], y_ref[sel[np.argmin(hi[sel])]],
               np.flatnonzero(rest)[np.argmax(lo[rest])], best_rest))
    # the order inside the list: each entry can be at least every later one
    later_lo = np.maximum.accumulate(lo[sel][::-1])[::-1]
    assert np.all(hi[sel][:-1] >= later_lo[1:]), "%s: list order contradicts the oracle" % what


TOPK_CASES = [(1, 1, 256, 1), (1, 5, 1024, 5), (1, 33, 96, 20), (1, 1000, 1024, 20),
              (1, 4099, 2560, 32), (1, 70001, 1024, 20), (1, 3000, 8192, 7),
              (2, 1000, 256, 20), (5, 4099, 1024, 1), (8, 70001, 2560, 20), (8, 64, 96, 32)]


@pytest.mark.parametrize("m,n,k,topk", TOPK_CASES, ids=["m%d-n%d-k%d-top%d" % c for c in TOPK_CASES])
def test_gemv_topk_selects_from_the_gemv_logits(q4, orc, m, n, k, topk):
    """The selection is exact on the kernel's own fp32 logits (those of q4_gemv, bit for
    bit), every logit is within tolerance of the oracle's, and the selection is a valid
    top-k of the oracle's products (assert_valid_topk)."""
    x, packed, scales, y_ref, bound = _case(orc, m, n, k, seed=m * 3 + n + k + topk)
    xg, pg, sg = gpu(x), gpu(packed), gpu(scales.view(np.float16))
    _log("q4_gemv_topk m=%d n=%d k=%d topk=%d" % (m, n, k, topk))
    values, rows = q4.q4_gemv_topk(xg, pg, sg, topk)
    logits = q4.q4_gemv(xg, pg, sg)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    vals, rws = values.cpu().numpy(), rows.cpu().numpy()
    # every logit of the kernel within tolerance of the oracle's
    assert_within(lg.astype(np.float64), y_ref, bound, "q4_gemv logits")
    for i in range(m):
        want = select_topk(lg[i], topk)
        assert np.array_equal(rws[i], want), "token %d rows %s != %s" % (i, rws[i][:8], want[:8])
        assert np.array_equal(vals[i].view(np.uint32), lg[i][want].view(np.uint32))
        assert_within(vals[i].astype(np.float64), y_ref[i][want], bound[i][want], "topk values")
        assert_valid_topk(rws[i], y_ref[i], bound[i], "token %d" % i)


@pytest.mark.parametrize("k", [512, 1024])
@pytest.mark.parametrize("delta", [-4, 0, 4])
def test_gemv1_second_wave_threshold(q4, orc, k, delta):
    """m = 1 at k <= 1024 runs a second wave per SIMD only when every wave gets two
    4-row steps or more, i.e. from 16 x CUs steps (n = 64 x CUs rows) on: rows on both
    sides of that switch (the grid, and so the number of top-k lists, changes there).
    Products against the oracle, the top-k selection against q4_gemv's logits and
    the oracle's products, and a two-matrix q4_gemv_multi whose rows together cross
    the switch, bit-identical to q4_gemv alone."""
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    n = 64 * cu + delta
    x, packed, scales, y_ref, bound = _case(orc, 1, n, k, seed=n + k)
    xg, pg, sg = gpu(x), gpu(packed), gpu(scales.view(np.float16))
    _log("q4_gemv / q4_gemv_topk m=1 n=%d k=%d (%d CUs)" % (n, k, cu))
    y = q4.q4_gemv(xg, pg, sg)
    values, rows = q4.q4_gemv_topk(xg, pg, sg, 20)
    torch.cuda.synchronize()
    lg = y.cpu().numpy()
    assert_within(lg.astype(np.float64), y_ref, bound, "q4_gemv")
    want = select_topk(lg[0], 20)
    assert np.array_equal(rows.cpu().numpy()[0], want)
    assert np.array_equal(values.cpu().numpy()[0].view(np.uint32), lg[0][want].view(np.uint32))
    assert_valid_topk(rows.cpu().numpy()[0], y_ref[0], bound[0], "topk")
    half = n // 2
    mats = [(pg[:half], sg[:half]), (pg[half:], sg[half:])]
    ys = q4.q4_gemv_multi(xg, mats)
    torch.cuda.synchronize()
    assert torch.equal(ys[0], y[:, :half]) and torch.equal(ys[1], y[:, half:])


@pytest.mark.parametrize("m,n", [(1, 300), (1, 5000), (3, 5000)])
def test_gemv_topk_ties(q4, orc, m, n):
    """Equal logits rank by row.  5000 equal rows exceed the candidate buffer
    of the final merge, so that case also takes its merge-everything route."""
    rng = np.random.default_rng(90 + n + m)
    k = 256
    base = (rng.standard_normal((1, k)) * 0.05).astype(np.float32)
    w = np.repeat(base, n, axis=0)                         # identical rows
    packed, scales = orc.quantize(w)
    x = rng.standard_normal((m, k)).astype(np.float16)
    _log("q4_gemv_topk ties m=%d n=%d" % (m, n))
    values, rows = q4.q4_gemv_topk(gpu(x), gpu(packed), gpu(scales.view(np.float16)), 32)
    for i in range(m):
        assert np.array_equal(rows.cpu().numpy()[i], np.arange(32))
        assert len(set(values.cpu().numpy()[i].tolist())) == 1


def test_gemv_topk_zero_weights(q4, orc):
    rng = np.random.default_rng(93)
    k = 256
    x = rng.standard_normal((1, k)).astype(np.float16)
    # all-zero weights: every logit is the same zero, so the rows tie
    zp, zs = orc.quantize(np.zeros((100, k), np.float32))
    values, rows = q4.q4_gemv_topk(gpu(x), gpu(zp), gpu(zs.view(np.float16)), 10)
    assert np.array_equal(rows.cpu().numpy()[0], np.arange(10))


def test_gemv_topk_deterministic_and_errors(q4, orc):
    x, packed, scales, _, _ = _case(orc, 1, 5000, 1024, seed=91)
    xg, pg, sg = gpu(x), gpu(packed), gpu(scales.view(np.float16))
    a = q4.q4_gemv_topk(xg, pg, sg, 20)
    b = q4.q4_gemv_topk(xg, pg, sg, 20)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    with pytest.raises(q4.Q4Error):
        q4.q4_gemv_topk(xg, pg, sg, 33)
    small = torch.empty(64, dtype=torch.uint8, device=DEV)
    with pytest.raises(q4.Q4Error) as err:
        q4.q4_gemv_topk(xg, pg, sg, 5, workspace=small)
    assert err.value.status == q4.Q4_ERR_WORKSPACE
    assert q4.q4_gemv_topk_workspace_size(1, 5000, 1024) > 0


@pytest.mark.parametrize("key,m,topk", [("decode_08b", 1, 20), ("decode_08b", 1, 1),
                                         ("decode_4b", 1, 20), ("decode_4b", 8, 20)])
def test_gemv_topk_lm_head_full_size(q4, orc, key, m, topk):
    """The full 248,320-row LM head: the fused selection equals the selection on
    q4_gemv's logits, every logit is within tolerance of the oracle's product
    (computed for all rows from the oracle's own quantization of the same
    generated weights), and the selection is a valid top-k of the oracle's
    products."""
    mat = qi.WORKLOADS[key].cases[-1][0]
    _log("topk %s m=%d: generating" % (mat.name, m))
    w = qi.weights(mat.n, mat.k, tensor_id=mat.tensor_id)
    packed, scales = q4.q4_quantize(gpu(w))
    rp, rs = orc.quantize(w)
    del w
    x = qi.activations(m, mat.k)
    xg = gpu(x)
    values, rows = q4.q4_gemv_topk(xg, packed, scales, topk)
    lg = q4.q4_gemv(xg, packed, scales).cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), rp), "codes differ from the oracle's"
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), rs), "scales differ"
    _log("topk %s m=%d: oracle product over all rows" % (mat.name, m))
    y_ref, bound = orc.matmul(x, rp, rs)
    assert_within(lg.astype(np.float64), y_ref, bound, "%s logits" % mat.name)
    for i in range(m):
        want = select_topk(lg[i], topk)
        assert np.array_equal(rows.cpu().numpy()[i], want)
        assert np.array_equal(values.cpu().numpy()[i].view(np.uint32), lg[i][want].view(np.uint32))
        assert_valid_topk(rows.cpu().numpy()[i], y_ref[i], bound[i], "%s token %d" % (mat.name, i))


# --------------------------------------------------------------------------
# fp16 weights (q4_gemv_f16)
# --------------------------------------------------------------------------

# k = 7168 is the largest k for which the m = 2..8 kernel that stages the activations and
# the weight tiles in LDS fits; 7200, 8192, 9120 and 16416 take the kernel that reads the
# activations from global memory.
F16_SHAPES = [(1, 32), (15, 64), (17, 96), (33, 256), (100, 1056), (257, 2560), (1024, 1024),
              (5, 8192), (61, 4096), (4099, 128), (9, 7168), (9, 7200), (9, 9120), (3, 16416)]


def _f16_case(m, n, k, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.05).astype(np.float16)
    x = (rng.standard_normal((m, k)) * 2).astype(np.float16)
    return x, w


@pytest.mark.parametrize("n,k", F16_SHAPES)
@pytest.mark.parametrize("m", [1, 2, 5, 8])
def test_gemv_f16_product(q4, orc, m, n, k):
    x, w = _f16_case(m, n, k, seed=m * 7 + n + k)
    _log("q4_gemv_f16 m=%d n=%d k=%d" % (m, n, k))
    y = q4.q4_gemv_f16(gpu(x), gpu(w))
    torch.cuda.synchronize()
    y_ref, bound = orc.matmul_f16(x, w)
    assert_within(y.cpu().numpy().astype(np.float64), y_ref, bound,
                  "q4_gemv_f16 m=%d n=%d k=%d" % (m, n, k))


@pytest.mark.parametrize("fn,m", [("q4_gemv_f16", 1), ("q4_gemv_f16", 8), ("q4_gemm_f16", 9),
                                  ("q4_gemm_f16", 33)])
def test_f16_longest_k(q4, orc, fn, m):
    """fp16 weights at the largest k the contract allows (2^24), n = 3."""
    n, k = 3, 2 ** 24
    x, w = _f16_case(m, n, k, seed=m + 24)
    _log("%s m=%d n=%d k=%d" % (fn, m, n, k))
    y = getattr(q4, fn)(gpu(x), gpu(w))
    torch.cuda.synchronize()
    y_ref, bound = orc.matmul_f16(x, w)
    assert_within(y.cpu().numpy().astype(np.float64), y_ref, bound, "%s k = 2^24" % fn)


def test_gemv_f16_exact_special_inputs(q4):
    rng = np.random.default_rng(78)
    n, k = 37, 96
    w = rng.standard_normal((n, k)).astype(np.float16)
    wg = gpu(w)
    _log("q4_gemv_f16 one-hot / zero inputs")
    for e0 in range(0, k, 8):
        x = np.eye(k, dtype=np.float16)[e0:e0 + 8]
        y = q4.q4_gemv_f16(gpu(x), wg).cpu().numpy().astype(np.float64)
        assert np.array_equal(y, w.astype(np.float64).T[e0:e0 + 8]), "one-hot rows %d.." % e0
    y = q4.q4_gemv_f16(gpu(np.zeros((3, k), np.float16)), wg)
    assert bool(torch.all(y == 0))
    y = q4.q4_gemv_f16(gpu(rng.standard_normal((2, k)).astype(np.float16)),
                       gpu(np.zeros((n, k), np.float16)))
    assert bool(torch.all(y == 0))


@pytest.mark.parametrize("k", [256, 2560, 4096])
def test_gemv_f16_single_token_one_hot(q4, k):
    """m = 1 streaming path (16, 32 and 64 lanes per row): a one-hot x picks one
    weight column exactly, for every position in a lane's chunks."""
    rng = np.random.default_rng(k)
    n = 70
    w = rng.standard_normal((n, k)).astype(np.float16)
    wg = gpu(w)
    _log("q4_gemv_f16 m=1 one-hot k=%d" % k)
    for e in list(range(0, 24)) + list(range(k - 24, k)) + list(rng.integers(0, k, 16)):
        x = np.zeros((1, k), np.float16)
        x[0, e] = 1.0
        y = q4.q4_gemv_f16(gpu(x), wg).cpu().numpy().astype(np.float64)
        assert np.array_equal(y[0], w[:, e].astype(np.float64)), "one-hot position %d" % e


def test_gemv_f16_deterministic_and_binding_errors(q4):
    x, w = _f16_case(8, 999, 2560, seed=6)
    xg, wg = gpu(x), gpu(w)
    a = q4.q4_gemv_f16(xg, wg)
    b = q4.q4_gemv_f16(xg, wg)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    with pytest.raises(q4.Q4Error):
        q4.q4_gemv_f16(gpu(np.zeros((9, 64), np.float16)), gpu(np.zeros((4, 64), np.float16)))
    with pytest.raises(ValueError):
        q4.q4_gemv_f16(gpu(np.zeros((1, 64), np.float16)), gpu(np.zeros((4, 32), np.float16)))


@pytest.mark.parametrize("mat,m", [(qi.DECODE_08B[-1], 1), (qi.DECODE_4B[-1], 8)],
                         ids=["lm_head_08b-m1", "lm_head_4b-m8"])
def test_gemv_f16_lm_head_full_size(q4, orc, mat, m):
    """The LM head in the fp16 format at full size: sampled rows against the oracle."""
    _log("f16 %s m=%d n=%d k=%d: generating" % (mat.name, m, mat.n, mat.k))
    w = qi.weights(mat.n, mat.k, tensor_id=mat.tensor_id).astype(np.float16)
    x = qi.activations(m, mat.k)
    y = q4.q4_gemv_f16(gpu(x), gpu(w))
    torch.cuda.synchronize()
    rows = _sample_rows(mat.n, np.random.default_rng(mat.tensor_id))
    y_ref, bound = orc.matmul_f16(x, w[rows])
    gy = y.cpu().numpy().astype(np.float64)[:, rows]
    assert_within(gy, y_ref, bound, "f16 %s" % mat.name)


# --------------------------------------------------------------------------
# fp16 weights, any m (q4_gemm_f16)
# --------------------------------------------------------------------------

F16_GEMM_SHAPES = [(15, 64), (17, 96), (100, 1056), (257, 2560), (61, 4096), (1000, 320)]


@pytest.mark.parametrize("n,k", F16_GEMM_SHAPES)
@pytest.mark.parametrize("m", [9, 16, 17, 32, 33, 64, 100, 255, 256, 300, 520, 1030])
def test_gemm_f16_product(q4, orc, m, n, k):
    x, w = _f16_case(m, n, k, seed=m * 11 + n + 3 * k)
    _log("q4_gemm_f16 m=%d n=%d k=%d" % (m, n, k))
    y = q4.q4_gemm_f16(gpu(x), gpu(w))
    torch.cuda.synchronize()
    y_ref, bound = orc.matmul_f16(x, w)
    assert_within(y.cpu().numpy().astype(np.float64), y_ref, bound,
                  "q4_gemm_f16 m=%d n=%d k=%d" % (m, n, k))


F16_TILING_CASES = [(64, 1000, 256), (100, 1000, 96), (256, 4096, 256), (250, 4090, 160),
                    (384, 4096, 128), (380, 4100, 96), (1030, 4096, 256), (768, 4100, 96),
                    (1000, 4000, 288), (2000, 4096, 64)]


@pytest.mark.parametrize("m,n,k", F16_TILING_CASES,
                         ids=["m%d-n%d-k%d" % c for c in F16_TILING_CASES])
def test_gemm_f16_every_tile_shape(q4, orc, m, n, k):
    """Shapes for which the fp16-weight GEMM picks each of its m > 32 tile
    shapes on a 256-CU device (32x64, 64x64, 64x128 and 128x128), each once
    with whole stages and once with a partial last stage (k / 32 not a
    multiple of the stage's groups) and ragged rows and columns, compared in
    full."""
    x, w = _f16_case(m, n, k, seed=m + n + k)
    _log("q4_gemm_f16 m=%d n=%d k=%d" % (m, n, k))
    y = q4.q4_gemm_f16(gpu(x), gpu(w))
    torch.cuda.synchronize()
    y_ref, bound = orc.matmul_f16(x, w)
    assert_within(y.cpu().numpy().astype(np.float64), y_ref, bound,
                  "q4_gemm_f16 m=%d n=%d k=%d" % (m, n, k))


def test_gemm_f16_exact_special_inputs(q4):
    """One-hot activation rows pick weight columns exactly; zero operands give zeros."""
    rng = np.random.default_rng(79)
    n, k = 70, 160
    w = rng.standard_normal((n, k)).astype(np.float16)
    wg = gpu(w)
    _log("q4_gemm_f16 one-hot / zero inputs")
    for m in (16, 40, 160):
        x = np.eye(k, dtype=np.float16)[:m]
        y = q4.q4_gemm_f16(gpu(x), wg).cpu().numpy().astype(np.float64)
        assert np.array_equal(y, w.astype(np.float64).T[:m]), "one-hot m=%d" % m
    y = q4.q4_gemm_f16(gpu(np.zeros((300, k), np.float16)), wg)
    assert bool(torch.all(y == 0))
    y = q4.q4_gemm_f16(gpu(rng.standard_normal((20, k)).astype(np.float16)),
                       gpu(np.zeros((n, k), np.float16)))
    assert bool(torch.all(y == 0))


def test_gemm_f16_deterministic_small_m_and_binding_errors(q4):
    x, w = _f16_case(300, 999, 2560, seed=8)
    xg, wg = gpu(x), gpu(w)
    a = q4.q4_gemm_f16(xg, wg)
    b = q4.q4_gemm_f16(xg, wg)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # m <= 8 is the decode kernel, bit for bit
    for m in (1, 8):
        assert torch.equal(q4.q4_gemm_f16(xg[:m], wg), q4.q4_gemv_f16(xg[:m], wg))
    with pytest.raises(ValueError):
        q4.q4_gemm_f16(gpu(np.zeros((9, 64), np.float16)), gpu(np.zeros((4, 32), np.float16)))
    with pytest.raises(q4.Q4Error):
        q4.q4_gemm_f16(gpu(np.zeros((9, 48), np.float16)), gpu(np.zeros((4, 48), np.float16)))


@pytest.mark.parametrize("m", [512, 2048])
def test_gemm_f16_prefill_full_size(q4, orc, m):
    """The 4B prefill projection (K=2560, N=4096) with fp16 weights at full size:
    sampled columns against the oracle on every token."""
    mat = qi.PREFILL_4B
    _log("f16 gemm %s m=%d n=%d k=%d: generating" % (mat.name, m, mat.n, mat.k))
    w = qi.weights(mat.n, mat.k, tensor_id=mat.tensor_id).astype(np.float16)
    x = qi.activations(m, mat.k, outliers=True)
    y = q4.q4_gemm_f16(gpu(x), gpu(w))
    torch.cuda.synchronize()
    rows = _sample_rows(mat.n, np.random.default_rng(mat.tensor_id), count=128)
    y_ref, bound = orc.matmul_f16(x, w[rows])
    gy = y.cpu().numpy().astype(np.float64)[:, rows]
    assert_within(gy, y_ref, bound, "f16 gemm %s m=%d" % (mat.name, m))


# --------------------------------------------------------------------------
# the five workload configurations at full size, compared in full
# --------------------------------------------------------------------------

def _sample_rows(n, rng, count=384):
    if n <= count:
        return np.arange(n)
    pick = rng.choice(n, count - 64, replace=False)
    return np.unique(np.concatenate([np.arange(32), np.arange(n - 32, n), pick]))


CASES = [(wl.key, i) for wl in qi.WORKLOADS.values() for i in range(len(wl.cases))]


@pytest.mark.parametrize("key,idx", CASES, ids=["%s-%d" % c for c in CASES])
def test_workload_full_size(q4, orc, key, idx):
    """Every code, scale and output of the configuration against the oracle,
    which quantizes the same generated weights itself and computes the whole
    product in fp64."""
    wl = qi.WORKLOADS[key]
    mat, m = wl.cases[idx]
    fn = "q4_gemv" if m <= 8 else "q4_gemm"
    _log("%s %s m=%d n=%d k=%d: generating" % (key, mat.name, m, mat.n, mat.k))
    w = qi.weights(mat.n, mat.k, tensor_id=mat.tensor_id, wide_groups=mat.wide_groups)
    x = qi.activations(m, mat.k, outliers=wl.outliers)
    wg = gpu(w)
    packed, scales = q4.q4_quantize(wg)
    del wg
    _log("%s: %s" % (mat.name, fn))
    y = getattr(q4, fn)(gpu(x), packed, scales)
    torch.cuda.synchronize()
    gp = packed.cpu().numpy()
    gs = scales.cpu().numpy().view(np.uint16)
    gy = y.cpu().numpy()
    del packed, scales, y
    _log("%s: oracle quantize + product over all rows" % mat.name)
    rp, rs = orc.quantize(w)
    del w
    assert np.array_equal(gs, rs), "scales differ from the oracle's"
    assert np.array_equal(gp, rp), "codes differ from the oracle's"
    y_ref, bound = orc.matmul(x, rp, rs)
    assert_within(gy.astype(np.float64), y_ref, bound, "%s %s" % (key, mat.name))


# --------------------------------------------------------------------------
# HIP graph capture: every entry point replayed from a graph
# --------------------------------------------------------------------------

def test_graph_replay_matches_eager(q4):
    """Every entry point captured once into a HIP graph (after eager calls, which also
    set the kernels' LDS attributes) and the graph replayed three times, with the outputs
    cleared and unrelated eager work and synchronizations between replays: every replay
    gives the eager results bit for bit (the kernels take no memset, and the top-k paths
    clear their own counters)."""
    rng = np.random.default_rng(2024)
    w1 = gpu((rng.standard_normal((4099, 2560)) * 0.02).astype(np.float32))
    w2 = gpu((rng.standard_normal((700, 1024)) * 0.02).astype(np.float32))
    wf = gpu((rng.standard_normal((1000, 1024)) * 0.02).astype(np.float16))
    x1 = gpu(rng.standard_normal((1, 2560)).astype(np.float16))
    x8 = gpu(rng.standard_normal((8, 2560)).astype(np.float16))
    x40 = gpu(rng.standard_normal((40, 1024)).astype(np.float16))
    x3 = gpu(rng.standard_normal((3, 1024)).astype(np.float16))
    p1, s1 = q4.q4_quantize(w1)
    p2, s2 = q4.q4_quantize(w2)
    torch.cuda.synchronize()
    outs = {
        "quantize": (torch.empty_like(p1), torch.empty_like(s1)),
        "gemv1": torch.empty((1, 4099), device=DEV),
        "gemv8": torch.empty((8, 4099), device=DEV),
        "multi1": [torch.empty((1, 4099), device=DEV), torch.empty((1, 2000), device=DEV)],
        "multi3": [torch.empty((3, 700), device=DEV), torch.empty((3, 300), device=DEV)],
        "gemm": torch.empty((40, 700), device=DEV),
        "gemm_multi": [torch.empty((40, 700), device=DEV), torch.empty((40, 300), device=DEV)],
        "topk1": (torch.empty((1, 20), device=DEV), torch.empty((1, 20), dtype=torch.int32, device=DEV)),
        "topk8": (torch.empty((8, 5), device=DEV), torch.empty((8, 5), dtype=torch.int32, device=DEV)),
        "noalloc": (torch.empty((1, 20), device=DEV), torch.empty((1, 20), dtype=torch.int32, device=DEV)),
        "gemv_f16": torch.empty((3, 1000), device=DEV),
        "gemm_f16": torch.empty((40, 1000), device=DEV),
    }
    ws1 = torch.empty(q4.q4_gemv_topk_workspace_size(1, 4099, 2560) + 256, dtype=torch.uint8, device=DEV)
    ws8 = torch.empty(q4.q4_gemv_topk_workspace_size(8, 4099, 2560) + 256, dtype=torch.uint8, device=DEV)

    def calls():
        q4.q4_quantize(w1, out=outs["quantize"])
        q4.q4_gemv(x1, p1, s1, out=outs["gemv1"])
        q4.q4_gemv(x8, p1, s1, out=outs["gemv8"])
        q4.q4_gemv_multi(x1, [(p1, s1), (p1[:2000], s1[:2000])], out=outs["multi1"])
        q4.q4_gemv_multi(x3, [(p2, s2), (p2[:300], s2[:300])], out=outs["multi3"])
        q4.q4_gemm(x40, p2, s2, out=outs["gemm"])
        q4.q4_gemm_multi(x40, [(p2, s2), (p2[:300], s2[:300])], out=outs["gemm_multi"])
        q4.q4_gemv_topk(x1, p1, s1, 20, workspace=ws1, out=outs["topk1"])
        q4.q4_gemv_topk(x8, p1, s1, 5, workspace=ws8, out=outs["topk8"])
        q4.q4_gemv_topk_noalloc(x1, p1, s1, 20, out=outs["noalloc"])
        q4.q4_gemv_f16(x3, wf, out=outs["gemv_f16"])
        q4.q4_gemm_f16(x40, wf, out=outs["gemm_f16"])

    def flat():
        res = []
        for v in outs.values():
            res.extend(v if isinstance(v, (list, tuple)) else [v])
        return res

    _log("graph capture of every entry point")
    calls()
    torch.cuda.synchronize()
    eager = [t.clone() for t in flat()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    scratch = torch.empty((8, 4099), device=DEV)
    for replay in range(3):
        for t in flat():
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(flat(), eager)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), \
                "replay %d: output %d differs from the eager call" % (replay, i)
        q4.q4_gemv(x8, p1, s1, out=scratch)            # unrelated eager work in between
        torch.cuda.synchronize()
