"""Seeded synthetic inputs for the attention workloads (no attention arithmetic here).

This module is shared by the tests, the benchmark and the smoke check; it only
draws random numbers and rounds them to the storage format.  It holds none of
the method's arithmetic and imports neither the HIP binding nor the oracle.

Draws: every tensor is i.i.d. standard normal from NumPy's PCG64 seeded with
``SeedSequence([seed, workload_id, tensor_id])`` (q=0, k=1, v=2, dO=3,
kv lengths=4), generated in float32 and, for bf16 storage, rounded to bf16 by
round-to-nearest-even bit arithmetic.  Both sides consume the same rounded
values: the GPU gets the bf16 bits, the oracle widens them exactly.

The workload shapes follow the probjax attention grids (batch 4, 8 heads,
head_dim 64/128, lengths 512..8192 and the non-tile-multiple 600/1500/3000),
the KV-length-masked case, the split-KV decode case, and the pages' GQA suite
(32 query heads, head_dim 128, batch 1, Lq = Lkv = T) and decode suite (32
query heads, head_dim 128, 8 or 32 KV heads, batch up to 8, up to 64k keys).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3, "kv_lens": 4}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    bits = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        bits[nan] = np.uint16(0x7FC0)
    return bits


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Case:
    """One attention problem: ``[B, T, H, D]`` tensors, GQA by head counts."""

    name: str
    B: int
    Tq: int
    Tkv: int
    Hq: int
    Hkv: int
    D: int
    dtype: str = "bf16"            # "bf16" or "fp32" storage of q, k, v, dO and outputs
    causal: bool = False
    kv_lens: Optional[Sequence[int]] = None   # fixed per-batch lengths, or None
    kv_len_range: Optional[tuple] = None      # (lo, hi) inclusive: draw lengths uniformly
    workload_id: int = 0                      # index into WORKLOADS, part of the seed
    decode: bool = False                      # few queries over a long KV cache
    window: Optional[tuple] = None            # local window (left, right), negative = no bound

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def replace(self, **kw) -> "Case":
        return dataclasses.replace(self, **kw)


def _rng(seed: int, workload_id: int, tensor: str) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, workload_id, TENSOR_IDS[tensor]]))


def normal_tensor(shape, seed: int, workload_id: int, tensor: str, dtype: str) -> np.ndarray:
    """i.i.d. N(0,1) draws: uint16 bf16 bits for ``dtype='bf16'``, float32 for ``'fp32'``."""
    x = _rng(seed, workload_id, tensor).standard_normal(size=shape, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "fp32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def draw_kv_lens(case: Case, seed: int = 0) -> Optional[np.ndarray]:
    """int32 ``[B]`` KV lengths: the fixed list, a uniform draw, or None (no mask)."""
    if case.kv_lens is not None:
        return np.asarray(case.kv_lens, dtype=np.int32)
    if case.kv_len_range is not None:
        lo, hi = case.kv_len_range
        return _rng(seed, case.workload_id, "kv_lens").integers(lo, hi, endpoint=True, size=case.B).astype(np.int32)
    return None


def make_inputs(case: Case, seed: int = 0, with_do: bool = True) -> dict:
    """Host arrays for one case: q, k, v (and dO) in storage format plus kv_lens."""
    qs = (case.B, case.Tq, case.Hq, case.D)
    ks = (case.B, case.Tkv, case.Hkv, case.D)
    out = {
        "q": normal_tensor(qs, seed, case.workload_id, "q", case.dtype),
        "k": normal_tensor(ks, seed, case.workload_id, "k", case.dtype),
        "v": normal_tensor(ks, seed, case.workload_id, "v", case.dtype),
        "kv_lens": draw_kv_lens(case, seed),
    }
    if with_do:
        out["do"] = normal_tensor(qs, seed, case.workload_id, "do", case.dtype)
    return out


def to_float64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of a storage-format array (bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


# The five workloads.  Index = workload_id used in the seed.
def workload_cases(workload_id: int) -> list:
    """All concrete cases of one workload, in a fixed order."""
    if workload_id == 0:   # fp32 correctness case
        return [Case("fp32_mha_T128_d64", 1, 128, 128, 2, 2, 64, "fp32", False, workload_id=0)]
    if workload_id == 1:   # bf16 d64 grid, tile-multiple and ragged lengths
        cases = []
        for t in (512, 1024, 2048, 600, 1500, 3000):
            for causal in (False, True):
                cases.append(Case(f"bf16_d64_T{t}_{'causal' if causal else 'full'}", 4, t, t, 8, 8, 64,
                                  "bf16", causal, workload_id=1))
        return cases
    if workload_id == 2:   # headline shape
        return [Case(f"bf16_d128_T8192_{'causal' if c else 'full'}", 4, 8192, 8192, 8, 8, 128, "bf16", c,
                     workload_id=2) for c in (False, True)]
    if workload_id == 3:   # KV-length mask
        return [Case("bf16_d128_T4096_kvlen", 4, 4096, 4096, 8, 8, 128, "bf16", False,
                     kv_lens=(1, 777, 2500, 4096), workload_id=3)]
    if workload_id == 4:   # split-KV GQA decode
        return [Case("bf16_gqa_decode_q16_kv16384", 4, 16, 16384, 32, 8, 128, "bf16", False,
                     kv_len_range=(1024, 16384), workload_id=4, decode=True)]
    if workload_id == 5:   # GQA suite: 32 query heads over 8 KV heads, batch 1, Lq = Lkv = T
        return [Case(f"bf16_gqa_suite_T{t}", 1, t, t, 32, 8, 128, "bf16", False, workload_id=5)
                for t in (1024, 2048, 4096, 8192, 16384)]
    if workload_id == 6:   # decode suite: one query per sequence over a full cache, 8 or 32 KV heads
        return [Case(f"bf16_decode_suite_B{b}_kv{n}_hkv{hkv}", b, 1, n, 32, hkv, 128, "bf16", False,
                     workload_id=6, decode=True)
                for hkv in (8, 32) for b in (1, 8) for n in (4096, 16384, 65536)]
    if workload_id == 7:   # headline shape with a causal sliding window of 1024 keys
        return [Case("bf16_d128_T8192_causal_window1024", 4, 8192, 8192, 8, 8, 128, "bf16", True,
                     window=(1024, 0), workload_id=7)]
    if workload_id == 8:   # fp32 grid: batch 4, 8 heads, head_dim 64 and 128
        return [Case(f"fp32_d{d}_T{t}_{'causal' if c else 'full'}", 4, t, t, 8, 8, d, "fp32", c, workload_id=8)
                for d in (64, 128) for t in (1024, 2048, 4096, 8192) for c in (False, True)]
    raise ValueError(f"no workload {workload_id}")


# Workloads 0-4 are the five configurations the parity tests cover in full
# (0: fp32 correctness case, 1: bf16 d64 grid, 2: headline, 3: KV-length
# mask, 4: GQA decode); 5 and 6 are the wider GQA and decode suites, 7 the
# local-window case, 8 the fp32 grid.
NUM_WORKLOADS = 9
