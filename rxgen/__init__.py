"""Seeded synthetic inputs shared by the tests and the benchmark.

This module draws input values only (see ``rxgen.c`` for the recipe); it
holds none of the arithmetic the library or the oracle compute. BF16 arrays
are returned as ``numpy.uint16`` bit patterns.

The named workloads below are the message shapes the library is measured
and checked on:

* ``flat_rank``: the usage example of the RCCLX article (code-journey.com,
  "Practical guide"): 8 ranks, a 10x20 FP32 tensor filled with the rank id,
  SUM allreduce -> every element is 0+1+...+7 = 28.
* ``flat_uniform``: the same shape with U[-1,1) values (seed 101).
* ``decode``: a decode-size allreduce, 8 BF16 buffers of 32x8192 = 262,144
  elements (512 KiB each), N(0,1) (seed 202).
* ``tree``: the DDA-tree per-rank step, 8 BF16 messages of 2,097,152 elements
  (4 MiB), N(0,1) (seed 303).
* ``lp_fp32``: low-precision allreduce, 8 FP32 inputs of 16,777,216 elements
  (64 MiB), N(0,1) with 1% outliers x100 (seed 404); E4M3, blocks of 128.
* ``lp_bf16``: low-precision large message, 8 BF16 inputs of 268,435,456
  elements (512 MiB), Laplace(0,1) (seed 505); E5M2, blocks of 256.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional

import numpy as np

FP32, BF16 = 0, 1
RANK, UNIFORM, NORMAL, NORMAL_OUTLIER, LAPLACE, INT = range(6)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "librxgen.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.rxg_fill.restype = ctypes.c_int
        lib.rxg_fill.argtypes = [
            ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
            ctypes.c_uint64, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64,
            ctypes.c_int]
        lib.rxg_mix.restype = ctypes.c_uint64
        lib.rxg_mix.argtypes = [ctypes.c_uint64]
        _lib = lib
    return _lib


def fill(count: int, dtype: int, dist: int, seed: int = 0, rank: int = 0,
         param: int = 0, offset: int = 0, nthreads: int = 0,
         out: Optional[np.ndarray] = None) -> np.ndarray:
    """Samples ``offset .. offset+count`` of stream (seed, rank).

    Returns float32 (FP32) or uint16 bit patterns (BF16)."""
    np_dtype = np.float32 if dtype == FP32 else np.uint16
    if out is None:
        out = np.empty(count, dtype=np_dtype)
    assert out.dtype == np_dtype and out.size == count and out.flags.c_contiguous
    rc = _load().rxg_fill(out.ctypes.data, count, dtype, dist, seed, rank,
                          param, offset, nthreads)
    if rc != 0:
        raise ValueError("rxg_fill rejected its arguments")
    return out


def mix(x: int) -> int:
    return int(_load().rxg_mix(x))


@dataclass(frozen=True)
class Workload:
    name: str
    op: str            # "flat", "tree" or "lp"
    nsrc: int
    count: int
    dtype: int         # FP32 or BF16
    dist: int
    seed: int
    fp8: Optional[str] = None   # "e4m3" / "e5m2" for the low-precision path
    block: Optional[int] = None

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == FP32 else 2

    def source(self, rank: int, offset: int = 0, count: Optional[int] = None,
               out: Optional[np.ndarray] = None) -> np.ndarray:
        n = self.count - offset if count is None else count
        return fill(n, self.dtype, self.dist, self.seed, rank, 0, offset,
                    out=out)

    def sources(self) -> List[np.ndarray]:
        return [self.source(r) for r in range(self.nsrc)]


WORKLOADS = {
    w.name: w for w in [
        Workload("flat_rank", "flat", 8, 200, FP32, RANK, 0),
        Workload("flat_uniform", "flat", 8, 200, FP32, UNIFORM, 101),
        Workload("decode", "flat", 8, 32 * 8192, BF16, NORMAL, 202),
        Workload("tree", "tree", 8, 2_097_152, BF16, NORMAL, 303),
        Workload("lp_fp32", "lp", 8, 16_777_216, FP32, NORMAL_OUTLIER, 404,
                 "e4m3", 128),
        Workload("lp_bf16", "lp", 8, 268_435_456, BF16, LAPLACE, 505,
                 "e5m2", 256),
    ]
}
