"""Checks on the gfx950 machine code of the library's own kernels (no GPU needed).

The device assembly of every source is generated with the same hipcc flags
the library is built with and scanned for two hazards:

* An MFMA inside a region where EXEC has been narrowed by a branch, with no
  ``s_cbranch_execz`` that skips the region when no lane is active.  Matrix
  instructions do not honour EXEC: a wave that reaches such an MFMA with every
  lane switched off still accumulates into its destination.  (This happened:
  a stage loop whose branch condition the compiler took for per-lane, with an
  unskipped two-MFMA block, gave wrong results for k = 64.)  Branches around
  MFMA code must be wave-uniform scalar branches or skipped regions.
* Packed fp32 VALU instructions (``v_pk_fma_f32``, ``v_pk_mul_f32``,
  ``v_pk_add_f32``): the library is built without them and must stay so.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from q4_group_quantized_amd import build as qb

HIPCC = qb.HIPCC if os.path.exists(qb.HIPCC) else shutil.which("hipcc")

_FUNC = re.compile(r"^(_Z[\w.$]+):")
_EXEC_DEST = re.compile(r"^s_\w+_b64\s+exec\s*,|^s_\w+_saveexec_b64\b")
_EXEC_RESTORE = re.compile(r"^s_(or|mov)_b64\s+exec\s*,")
_PACKED_F32 = re.compile(r"^v_pk_(fma|mul|add)_f32\b")


def masked_mfma_hits(asm_text):
    """(function, line) of every MFMA in an exec-narrowed, unskipped region."""
    fn, masked, skipped, hits = None, False, False, []
    after_jump = False
    for ln, line in enumerate(asm_text.splitlines(), 1):
        t = line.strip()
        if not t or t.startswith(";"):
            continue
        m = _FUNC.match(t)
        if m:
            fn, masked, skipped, after_jump = m.group(1), False, False, False
            continue
        if t.startswith(".LBB"):
            # a block that follows an unconditional jump is entered only by a
            # branch: its mask state is not the one scanned so far
            if after_jump:
                masked, skipped = False, False
            continue
        after_jump = t.startswith("s_branch") or t.startswith("s_endpgm") or \
            t.startswith("s_setpc")
        if _EXEC_RESTORE.match(t):
            masked = False
            continue
        if _EXEC_DEST.match(t):
            masked, skipped = True, False
            continue
        if masked and t.startswith("s_cbranch_execz"):
            skipped = True
            continue
        if masked and not skipped and t.startswith("v_mfma"):
            hits.append((fn, ln))
    return hits


def test_scanner_flags_an_unskipped_masked_mfma():
    bad = "\n".join([
        "_Zk:",
        "v_cmp_lt_i32_e32 vcc, v1, v2",
        "s_and_saveexec_b64 s[2:3], vcc",
        "v_mfma_f32_16x16x32_f16 v[2:5], v[6:9], v[10:13], v[2:5]",
        "s_or_b64 exec, exec, s[2:3]",
    ])
    good = bad.replace("s_and_saveexec_b64 s[2:3], vcc",
                       "s_and_saveexec_b64 s[2:3], vcc\ns_cbranch_execz .LBB0_2")
    assert masked_mfma_hits(bad) == [("_Zk", 4)]
    assert masked_mfma_hits(good) == []
    assert masked_mfma_hits(bad.replace("s_and_saveexec_b64 s[2:3], vcc",
                                        "s_and_b64 exec, exec, vcc")) == [("_Zk", 4)]


def _device_asm(src):
    out = os.path.join(qb.BUILD_DIR, "lint_" + os.path.splitext(src)[0] + ".s")
    cmd = [HIPCC, *[f for f in qb.FLAGS if f != "-fPIC"], "--cuda-device-only", "-S",
           os.path.join(qb.CSRC, src), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc -S failed for %s:\n%s" % (src, res.stderr))
    with open(out) as f:
        return f.read()


@pytest.mark.skipif(HIPCC is None, reason="hipcc not available")
def test_library_kernels_have_no_masked_mfma_and_no_packed_fp32():
    os.makedirs(qb.BUILD_DIR, exist_ok=True)
    srcs = [s for s in qb.SOURCES if s != "q4_api.hip"]
    with ThreadPoolExecutor(max_workers=4) as ex:
        asms = dict(zip(srcs, ex.map(_device_asm, srcs)))
    mfma_total = 0
    for src, asm in asms.items():
        mfma_total += sum(1 for l in asm.splitlines() if l.strip().startswith("v_mfma"))
        hits = masked_mfma_hits(asm)
        assert not hits, "%s: MFMA under a narrowed EXEC without a skip at %s" % (src, hits[:4])
        packed = [l.strip() for l in asm.splitlines() if _PACKED_F32.match(l.strip())]
        assert not packed, "%s: packed fp32 instructions %s" % (src, packed[:4])
    assert mfma_total > 0              # the scan saw the matrix kernels
