"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no step of the quantizer or of the product: it only draws
random numbers with numpy's PCG64 and shapes them like the workloads the pages
describe.  Both the GPU path and the CPU oracle receive the same arrays.

Shapes come from the model tables of the two QORA pages (hidden size 1024 and
2560, DeltaNet heads of 128, attention heads of 256, a 248,320-token
vocabulary): QORA-LLM-0.8B model card, "Architecture"; QORA-4B forum article,
model specification table.  There are no trained weights: weights are drawn
from N(0, 0.02^2) and activations from N(0, 1).

Streams: every tensor has its own generator ``default_rng([seed, tensor_id,
chunk])`` so that any row range can be regenerated independently.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

ROW_CHUNK = 4096          # weights are drawn in blocks of this many rows
W_STD = np.float32(0.02)
WIDE_GROUP_EVERY = 64     # "wide-scale" weights: every 64th group of 32 ...
WIDE_GROUP_FACTOR = np.float32(10.0)   # ... is multiplied by 10
OUTLIER_FRACTION = 0.01   # activations: 1% of the input channels ...
OUTLIER_FACTOR = np.float32(20.0)      # ... are multiplied by 20

VOCAB = 248320


def weight_rows(n: int, k: int, row0: int, row1: int, *, seed: int = 0,
                tensor_id: int = 0, wide_groups: bool = False) -> np.ndarray:
    """Rows [row0, row1) of a synthetic fp32 weight matrix W [n, k]."""
    if not (0 <= row0 <= row1 <= n):
        raise ValueError("bad row range")
    out = np.empty((row1 - row0, k), dtype=np.float32)
    c0, c1 = row0 // ROW_CHUNK, (row1 + ROW_CHUNK - 1) // ROW_CHUNK
    for c in range(c0, c1):
        lo, hi = c * ROW_CHUNK, min((c + 1) * ROW_CHUNK, n)
        rng = np.random.default_rng([seed, tensor_id, c])
        block = rng.standard_normal((hi - lo, k), dtype=np.float32)
        block *= W_STD
        a, b = max(lo, row0), min(hi, row1)
        out[a - row0:b - row0] = block[a - lo:b - lo]
    if wide_groups:
        # flat row-major group index g = row * (k // 32) + j; g % 64 == 0 -> x10
        gpr = k // 32
        flat0 = row0 * gpr
        groups = out.reshape(-1, 32)
        first = (-flat0) % WIDE_GROUP_EVERY
        groups[first::WIDE_GROUP_EVERY] *= WIDE_GROUP_FACTOR
    return out


def weights(n: int, k: int, *, seed: int = 0, tensor_id: int = 0,
            wide_groups: bool = False) -> np.ndarray:
    """A whole synthetic fp32 weight matrix W [n, k]."""
    return weight_rows(n, k, 0, n, seed=seed, tensor_id=tensor_id,
                       wide_groups=wide_groups)


def outlier_channels(k: int, *, seed: int = 0, tensor_id: int = 1000) -> np.ndarray:
    """round(1% of k) input channels, from a seeded permutation."""
    cnt = int(round(OUTLIER_FRACTION * k))
    rng = np.random.default_rng([seed, tensor_id, 0])
    return np.sort(rng.permutation(k)[:cnt])


def activations(m: int, k: int, *, seed: int = 0, tensor_id: int = 999,
                outliers: bool = False) -> np.ndarray:
    """Synthetic fp16 activations x [m, k] ~ N(0,1) (numpy's fp16 cast).

    With ``outliers`` the same 1% of channels is scaled by 20 in every row,
    in fp32, before the cast to fp16."""
    rng = np.random.default_rng([seed, tensor_id, 0])
    x = rng.standard_normal((m, k), dtype=np.float32)
    if outliers:
        x[:, outlier_channels(k, seed=seed)] *= OUTLIER_FACTOR
    return x.astype(np.float16)


# --------------------------------------------------------------------------
# Workload registry: the five problem configurations.
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Matrix:
    name: str
    n: int
    k: int
    tensor_id: int
    wide_groups: bool = False


@dataclass(frozen=True)
class Workload:
    """A named set of products; each case is (matrix, m)."""
    key: str
    description: str
    cases: Tuple[Tuple[Matrix, int], ...]
    outliers: bool = False


def _set(prefix: str, k: int, shapes: Sequence[Tuple[str, int]],
         wide: bool = False, base_id: int = 0) -> Tuple[Matrix, ...]:
    return tuple(Matrix("%s.%s" % (prefix, nm), n, k, base_id + i, wide)
                 for i, (nm, n) in enumerate(shapes))


# 0.8B (hidden 1024): DeltaNet 16 QK heads and 16 V heads of 128; attention
# 8 query heads and 2 KV heads of 256; LM head over the 248,320-token vocab.
DECODE_08B = _set("08b", 1024, [
    ("deltanet_q", 2048), ("deltanet_k", 2048), ("deltanet_v", 2048),
    ("attn_q", 2048), ("attn_k", 512), ("attn_v", 512), ("lm_head", VOCAB)],
    base_id=100)

# 4B (hidden 2560): DeltaNet 16 QK heads and 32 V heads of 128; attention
# 16 query heads and 4 KV heads of 256; LM head over the same vocabulary.
DECODE_4B = _set("4b", 2560, [
    ("deltanet_q", 2048), ("deltanet_k", 2048), ("deltanet_v", 4096),
    ("attn_q", 4096), ("attn_k", 1024), ("attn_v", 1024), ("lm_head", VOCAB)],
    base_id=200)

PREFILL_4B = Matrix("4b.prefill", 4096, 2560, 300)
LM_HEAD_4B_WIDE = Matrix("4b.lm_head_wide", VOCAB, 2560, 400, True)
PREFILL_4B_WIDE = Matrix("4b.prefill_wide", 4096, 2560, 401, True)

WORKLOADS: Dict[str, Workload] = {
    "single": Workload(
        "single", "single GEMV M=1, K=1024, N=1024",
        ((Matrix("single", 1024, 1024, 0), 1),)),
    "decode_08b": Workload(
        "decode_08b", "0.8B-shaped decode set, M=1, K=1024",
        tuple((mat, 1) for mat in DECODE_08B)),
    "decode_4b": Workload(
        "decode_4b", "4B-shaped decode set, M=1, K=2560",
        tuple((mat, 1) for mat in DECODE_4B)),
    "prefill_4b": Workload(
        "prefill_4b", "4B-shaped prefill GEMM, K=2560, N=4096, 1% outlier channels x20",
        ((PREFILL_4B, 16), (PREFILL_4B, 128), (PREFILL_4B, 512)), outliers=True),
    "verify_long_4b": Workload(
        "verify_long_4b",
        "speculative-verify LM head M=8 and long prefill M=2048, every 64th group x10",
        ((LM_HEAD_4B_WIDE, 8), (PREFILL_4B_WIDE, 2048))),
}


def workload_bytes(m: int, n: int, k: int) -> int:
    """Algorithmic HBM bytes of one product: packed + scales + x + y."""
    return n * k // 2 + n * (k // 32) * 2 + 2 * m * k + 4 * m * n


def workload_flops(m: int, n: int, k: int) -> int:
    return 2 * m * n * k
