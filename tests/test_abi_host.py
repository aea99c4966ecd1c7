"""Host-side checks of the C ABI library (no GPU needed, nothing is launched).

The library must load, export every entry point include/q4.h declares, and
reject invalid arguments on the host before touching the device.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q4_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import q4_group_quantized_amd as q4
    if not os.path.exists(q4.LIB_PATH):
        from q4_group_quantized_amd import build
        build.build()
    return q4.load()


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for fn in ("q4_quantize", "q4_gemv", "q4_gemm", "q4_status_str", "q4_abi_version"):
        assert fn in names


def test_library_exports_every_declared_symbol(lib):
    import q4_group_quantized_amd as q4
    out = subprocess.run(["nm", "-D", "--defined-only", q4.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (q4_[a-z0-9_]+)\b", out))
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing
    for f in declared_functions():
        getattr(lib, f)


def test_version_and_status_strings(lib):
    m = re.search(r"#define Q4_ABI_VERSION (\d+)", open(HEADER).read())
    assert lib.q4_abi_version() == int(m.group(1))
    seen = set()
    for code in range(8):
        s = lib.q4_status_str(code).decode()
        assert s and s not in seen
        seen.add(s)
    assert lib.q4_status_str(99).decode() == "unknown status"


FAKE = 0x10000          # never dereferenced: validation fails before any use
NULL = None


@pytest.mark.parametrize("args,expect", [
    ((NULL, FAKE, FAKE, 4, 64), 1),
    ((FAKE, NULL, FAKE, 4, 64), 1),
    ((FAKE, FAKE, NULL, 4, 64), 1),
    ((FAKE, FAKE, FAKE, 0, 64), 2),
    ((FAKE, FAKE, FAKE, 4, 16), 2),
    ((FAKE, FAKE, FAKE, 4, 48), 2),
    ((FAKE, FAKE, FAKE, 2 ** 31, 64), 2),
    ((FAKE, FAKE, FAKE, 4, 2 ** 24 + 32), 2),
    ((FAKE, FAKE, FAKE, 2 ** 20, 2 ** 21), 2),
    ((FAKE + 4, FAKE, FAKE, 4, 64), 3),
    ((FAKE, FAKE + 8, FAKE, 4, 64), 3),
    ((FAKE, FAKE, FAKE + 1, 4, 64), 3),
])
def test_quantize_rejects_bad_arguments(lib, args, expect):
    assert lib.q4_quantize(*args, None) == expect


@pytest.mark.parametrize("fn", ["q4_gemv", "q4_gemm"])
@pytest.mark.parametrize("args,expect", [
    ((NULL, FAKE, FAKE, FAKE, 1, 8, 64), 1),
    ((FAKE, NULL, FAKE, FAKE, 1, 8, 64), 1),
    ((FAKE, FAKE, NULL, FAKE, 1, 8, 64), 1),
    ((FAKE, FAKE, FAKE, NULL, 1, 8, 64), 1),
    ((FAKE, FAKE, FAKE, FAKE, 0, 8, 64), 2),
    ((FAKE, FAKE, FAKE, FAKE, 1, 0, 64), 2),
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, 0), 2),
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, 33), 2),
    ((FAKE, FAKE, FAKE, FAKE, -3, 8, 64), 2),
    ((FAKE + 2, FAKE, FAKE, FAKE, 1, 8, 64), 3),
    ((FAKE, FAKE + 4, FAKE, FAKE, 1, 8, 64), 3),
    ((FAKE, FAKE, FAKE + 1, FAKE, 1, 8, 64), 3),
    ((FAKE, FAKE, FAKE, FAKE + 2, 1, 8, 64), 3),
])
def test_products_reject_bad_arguments(lib, fn, args, expect):
    assert getattr(lib, fn)(*args, None) == expect


def test_gemv_rejects_more_than_eight_rows(lib):
    assert lib.q4_gemv(FAKE, FAKE, FAKE, FAKE, 9, 8, 64, None) == 2


@pytest.mark.parametrize("args,expect", [
    ((NULL, FAKE, FAKE, 1, 8, 64), 1),
    ((FAKE, NULL, FAKE, 1, 8, 64), 1),
    ((FAKE, FAKE, NULL, 1, 8, 64), 1),
    ((FAKE, FAKE, FAKE, 0, 8, 64), 2),
    ((FAKE, FAKE, FAKE, 9, 8, 64), 2),
    ((FAKE, FAKE, FAKE, 1, 0, 64), 2),
    ((FAKE, FAKE, FAKE, 1, 8, 48), 2),
    ((FAKE, FAKE, FAKE, 1, 8, 16), 2),
    ((FAKE + 2, FAKE, FAKE, 1, 8, 64), 3),
    ((FAKE, FAKE + 8, FAKE, 1, 8, 64), 3),
    ((FAKE, FAKE, FAKE + 2, 1, 8, 64), 3),
])
def test_gemv_f16_rejects_bad_arguments(lib, args, expect):
    assert lib.q4_gemv_f16(*args, None) == expect


@pytest.mark.parametrize("args,expect", [
    ((NULL, FAKE, FAKE, 16, 8, 64), 1),
    ((FAKE, NULL, FAKE, 16, 8, 64), 1),
    ((FAKE, FAKE, NULL, 16, 8, 64), 1),
    ((FAKE, FAKE, FAKE, 0, 8, 64), 2),
    ((FAKE, FAKE, FAKE, -3, 8, 64), 2),
    ((FAKE, FAKE, FAKE, 1 << 31, 8, 64), 2),
    ((FAKE, FAKE, FAKE, 16, 0, 64), 2),
    ((FAKE, FAKE, FAKE, 16, 8, 48), 2),
    ((FAKE, FAKE, FAKE, 16, 8, 16), 2),
    ((FAKE + 2, FAKE, FAKE, 16, 8, 64), 3),
    ((FAKE, FAKE + 8, FAKE, 16, 8, 64), 3),
    ((FAKE, FAKE, FAKE + 2, 16, 8, 64), 3),
])
def test_gemm_f16_rejects_bad_arguments(lib, args, expect):
    # argument checks run before the device check, so a GPU-less host sees them
    assert lib.q4_gemm_f16(*args, None) == expect


@pytest.mark.parametrize("args,expect", [
    ((NULL, FAKE, FAKE, 1, 64, 64, 5, FAKE, FAKE, FAKE, 1 << 20), 1),
    ((FAKE, NULL, FAKE, 1, 64, 64, 5, FAKE, FAKE, FAKE, 1 << 20), 1),
    ((FAKE, FAKE, NULL, 1, 64, 64, 5, FAKE, FAKE, FAKE, 1 << 20), 1),
    ((FAKE, FAKE, FAKE, 1, 64, 64, 5, NULL, FAKE, FAKE, 1 << 20), 1),
    ((FAKE, FAKE, FAKE, 1, 64, 64, 5, FAKE, NULL, FAKE, 1 << 20), 1),
    ((FAKE, FAKE, FAKE, 0, 64, 64, 5, FAKE, FAKE, FAKE, 1 << 20), 2),
    ((FAKE, FAKE, FAKE, 9, 64, 64, 5, FAKE, FAKE, FAKE, 1 << 20), 2),
    ((FAKE, FAKE, FAKE, 1, 64, 64, 0, FAKE, FAKE, FAKE, 1 << 20), 2),
    ((FAKE, FAKE, FAKE, 1, 64, 64, 33, FAKE, FAKE, FAKE, 1 << 20), 2),
    ((FAKE, FAKE, FAKE, 1, 4, 64, 5, FAKE, FAKE, FAKE, 1 << 20), 2),
    ((FAKE, FAKE, FAKE, 1, 64, 48, 5, FAKE, FAKE, FAKE, 1 << 20), 2),
    ((FAKE + 2, FAKE, FAKE, 1, 64, 64, 5, FAKE, FAKE, FAKE, 1 << 20), 3),
    ((FAKE, FAKE, FAKE, 1, 64, 64, 5, FAKE + 2, FAKE, FAKE, 1 << 20), 3),
    ((FAKE, FAKE, FAKE, 1, 64, 64, 5, FAKE, FAKE + 1, FAKE, 1 << 20), 3),
])
def test_gemv_topk_rejects_bad_arguments(lib, args, expect):
    # argument checks run before the device check, so a GPU-less host sees them
    assert lib.q4_gemv_topk(*args, None) == expect


@pytest.mark.parametrize("args,expect", [
    ((NULL, FAKE, FAKE, 1, 64, 64, 5, FAKE, FAKE), 1),
    ((FAKE, FAKE, FAKE, 1, 64, 64, 5, NULL, FAKE), 1),
    ((FAKE, FAKE, FAKE, 9, 64, 64, 5, FAKE, FAKE), 2),
    ((FAKE, FAKE, FAKE, 1, 64, 64, 33, FAKE, FAKE), 2),
    ((FAKE, FAKE, FAKE, 1, 64, 48, 5, FAKE, FAKE), 2),
    ((FAKE + 2, FAKE, FAKE, 1, 64, 64, 5, FAKE, FAKE), 3),
])
def test_gemv_topk_noalloc_rejects_bad_arguments(lib, args, expect):
    # the no-allocation form runs the same host checks first
    assert lib.q4_gemv_topk_noalloc(*args, None) == expect


def test_gemv_topk_workspace_size_without_device(lib):
    assert lib.q4_gemv_topk_workspace_size(1, 64, 48) == 0      # invalid shape


def _multi(lib, x, m, k, packed, scales, y, n, count=None, fn="q4_gemv_multi"):
    """Call q4_gemv_multi (or q4_gemm_multi) with host arrays built from Python lists
    (None = NULL array)."""
    def arr(vals, ctype):
        return None if vals is None else (ctype * max(len(vals), 1))(*vals)
    cnt = len(n) if count is None else count
    return getattr(lib, fn)(x, m, k, cnt, arr(packed, ctypes.c_void_p),
                             arr(scales, ctypes.c_void_p), arr(y, ctypes.c_void_p),
                             arr(n, ctypes.c_int64), None)


@pytest.mark.parametrize("case,expect", [
    (dict(packed=None), 1),
    (dict(scales=None), 1),
    (dict(y=None), 1),
    (dict(n=None, count=2), 1),
    (dict(x=None), 1),
    (dict(packed=[FAKE, NULL]), 1),
    (dict(scales=[NULL, FAKE]), 1),
    (dict(y=[FAKE, NULL]), 1),
    (dict(count=0), 2),
    (dict(count=9, packed=[FAKE] * 9, scales=[FAKE] * 9, y=[FAKE] * 9, n=[8] * 9), 2),
    (dict(count=-1), 2),
    (dict(m=0), 2),
    (dict(m=9), 2),
    (dict(k=48), 2),
    (dict(n=[8, 0]), 2),
    (dict(n=[8, 2 ** 31]), 2),
    (dict(x=FAKE + 2), 3),
    (dict(packed=[FAKE, FAKE + 4]), 3),
    (dict(scales=[FAKE + 1, FAKE]), 3),
    (dict(y=[FAKE, FAKE + 2]), 3),
])
def test_gemv_multi_rejects_bad_arguments(lib, case, expect):
    args = dict(x=FAKE, m=1, k=64, packed=[FAKE, FAKE], scales=[FAKE, FAKE], y=[FAKE, FAKE],
                n=[8, 8], count=None)
    args.update(case)
    assert _multi(lib, **args) == expect


@pytest.mark.parametrize("case,expect", [
    (dict(packed=None), 1),
    (dict(y=[FAKE, NULL]), 1),
    (dict(count=0), 2),
    (dict(count=9, packed=[FAKE] * 9, scales=[FAKE] * 9, y=[FAKE] * 9, n=[8] * 9), 2),
    (dict(m=0), 2),
    (dict(k=48), 2),
    (dict(n=[8, 0]), 2),
    (dict(x=FAKE + 2), 3),
    (dict(scales=[FAKE + 1, FAKE]), 3),
])
def test_gemm_multi_rejects_bad_arguments(lib, case, expect):
    args = dict(x=FAKE, m=40, k=64, packed=[FAKE, FAKE], scales=[FAKE, FAKE], y=[FAKE, FAKE],
                n=[8, 8], count=None)
    args.update(case)
    assert _multi(lib, **args, fn="q4_gemm_multi") == expect


def test_binding_names_match_the_c_abi():
    import q4_group_quantized_amd as q4
    for name in ("q4_quantize", "q4_gemv", "q4_gemm", "q4_gemv_multi", "q4_gemm_multi",
                 "q4_gemv_f16",
                 "q4_gemv_topk", "q4_gemv_topk_workspace_size", "q4_gemv_topk_noalloc",
                 "q4_status_str",
                 "q4_abi_version"):
        assert callable(getattr(q4, name))
    assert set(q4.EXPORTED) == set(declared_functions())
