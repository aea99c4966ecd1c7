"""q4_gemv_topk_noalloc (the entry point that allocates nothing) against
q4_gemv_topk with a caller workspace: the same kernels, so the same bits.

Two calls in a row on the library's scratch buffer, the second on a smaller
problem, so that it runs over what the first one left there; plus the size
limit of that buffer.
"""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _log(msg):
    print("[no-alloc] " + msg, flush=True)


@pytest.fixture(scope="module")
def q4():
    import q4_group_quantized_amd as mod
    assert torch.cuda.is_available(), "GPU tests need a device"
    mod.load()
    return mod


def _problem(orc, m, n, k, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = (rng.standard_normal((m, k)) * 2).astype(np.float16)
    packed, scales = orc.quantize(w)
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return g(x), g(packed), g(scales.view(np.float16))


# (m, n, k, topk) pairs: the second problem of each pair is smaller than the
# first, and the pairs cover the fused m = 1 path and the product + scan path
PAIRS = [((8, 70001, 2560, 20), (1, 5000, 1024, 5)),
         ((1, 248320, 1024, 20), (3, 4099, 256, 32)),
         ((5, 30000, 1024, 7), (2, 1000, 96, 1))]


@pytest.mark.parametrize("first,second", PAIRS, ids=["pair%d" % i for i in range(len(PAIRS))])
def test_noalloc_matches_workspace_form(q4, first, second):
    orc = oracle.get()
    for i, (m, n, k, topk) in enumerate((first, second)):
        _log("call %d: m=%d n=%d k=%d topk=%d" % (i, m, n, k, topk))
        x, p, s = _problem(orc, m, n, k, seed=m * 131 + n + k + topk)
        v_ref, r_ref = q4.q4_gemv_topk(x, p, s, topk)
        v, r = q4.q4_gemv_topk_noalloc(x, p, s, topk)
        torch.cuda.synchronize()
        assert torch.equal(r, r_ref), "rows differ on call %d" % i
        assert torch.equal(v.view(torch.int32), v_ref.view(torch.int32)), \
            "values differ on call %d" % i


def test_noalloc_rejects_problems_beyond_its_buffer(q4):
    # m = 8 over 600,000 rows needs 19.2 MB of logits: more than the 16 MiB buffer
    m, n, k = 8, 600000, 256
    need = q4.q4_gemv_topk_workspace_size(m, n, k)
    assert need > q4.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((m, k), dtype=torch.float16, device=DEV)
    p = torch.zeros((n, k // 2), dtype=torch.uint8, device=DEV)
    s = torch.zeros((n, k // 32), dtype=torch.float16, device=DEV)
    with pytest.raises(q4.Q4Error) as err:
        q4.q4_gemv_topk_noalloc(x, p, s, 4)
    assert err.value.status == q4.Q4_ERR_TOO_LARGE
    # the largest workload of the path fits: the 248,320-row LM head at m = 8
    assert q4.q4_gemv_topk_workspace_size(8, 248320, 2560) <= q4.NOALLOC_SCRATCH_BYTES
