"""ctypes view of the CPU oracle (``rx_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and
the benchmark's CPU-baseline leg; the product path never imports it.

Arrays are numpy: FP32 as float32, BF16 as uint16 bit patterns, FP8 codes as
uint8, scales as float32.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import numpy as np

FP32, BF16, E4M3, E5M2 = 0, 1, 2, 3
DRR_SUM, DRR_REQUANT = 0, 1
ALGO_FLAT, ALGO_TREE, ALGO_LOWPREC = 1, 2, 3
FMT = {"e4m3": E4M3, "e5m2": E5M2}

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librxoracle.so")
_lib = None

_P = ctypes.c_void_p
_SZ = ctypes.c_size_t
_I = ctypes.c_int


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "rxo_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
            "rxo_f32_to_bf16": (ctypes.c_uint16, [ctypes.c_float]),
            "rxo_fp8_max": (ctypes.c_float, [_I]),
            "rxo_fp8_decode": (ctypes.c_float, [ctypes.c_uint8, _I]),
            "rxo_fp8_encode": (ctypes.c_uint8, [ctypes.c_float, _I]),
            "rxo_fp8_encode_array": (None, [_P, _SZ, _I, _P]),
            "rxo_fp8_encode_bits_range": (None, [ctypes.c_uint32, ctypes.c_uint32, _I, _P]),
            "rxo_f32_to_bf16_array": (None, [_P, _SZ, _P]),
            "rxo_fp8_decode_array": (None, [_P, _SZ, _I, _P]),
            "rxo_block_scale": (None, [_P, _SZ, _I, _P, _P]),
            "rxo_block_scale_bits_range": (None, [ctypes.c_uint32, ctypes.c_uint32, _I, _P, _P]),
            "rxo_reduce_flat": (None, [_P, _I, _SZ, _I, _P]),
            "rxo_tree_chunk": (None, [_SZ, _I, _I, _I, _P, _P]),
            "rxo_reduce_scatter_chunk_bcast": (None, [_P, _I, _SZ, _I, _I, _P]),
            "rxo_quant_fp8": (None, [_P, _I, _SZ, _I, _I, _I, _P, _P]),
            "rxo_dequant_reduce_requant": (None, [_P, _P, _I, _SZ, _I, _I, _I,
                                                  _P, _P, _P, _I]),
            "rxo_lp_tree_chunk": (None, [_SZ, _I, _I, _I, _P, _P]),
            "rxo_allreduce_local": (None, [_P, _I, _SZ, _I, _I, _I, _I]),
            "rxo_lp_reduce_scatter_chunk_bcast": (None, [_P, _P, _I, _SZ, _I, _I, _I,
                                                         _P, _P, _P, _I]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptrs(arrays: Sequence[np.ndarray]):
    arr = (ctypes.c_void_p * len(arrays))(*[a.ctypes.data for a in arrays])
    return arr


def _np_of(dtype: int):
    return np.float32 if dtype == FP32 else np.uint16


def _check(arrays: Sequence[np.ndarray], np_dtype, count: Optional[int] = None):
    for a in arrays:
        assert a.dtype == np_dtype and a.flags.c_contiguous, (a.dtype, np_dtype)
        if count is not None:
            assert a.size >= count


# ---- scalar codecs -------------------------------------------------------

def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.size, dtype=np.uint16)
    lib().rxo_f32_to_bf16_array(x.ctypes.data, x.size, out.ctypes.data)
    return out.reshape(x.shape)


def fp8_max(fmt: int) -> float:
    return float(lib().rxo_fp8_max(fmt))


def fp8_encode(x: np.ndarray, fmt: int) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.size, dtype=np.uint8)
    lib().rxo_fp8_encode_array(x.ctypes.data, x.size, fmt, out.ctypes.data)
    return out.reshape(x.shape)


def fp8_encode_bits(first: int, n: int, fmt: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8)
    lib().rxo_fp8_encode_bits_range(first, n, fmt, out.ctypes.data)
    return out


def fp8_decode(c: np.ndarray, fmt: int) -> np.ndarray:
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.size, dtype=np.float32)
    lib().rxo_fp8_decode_array(c.ctypes.data, c.size, fmt, out.ctypes.data)
    return out.reshape(c.shape)


def block_scale(x: np.ndarray, fmt: int) -> Tuple[float, float]:
    x = np.ascontiguousarray(x, dtype=np.float32)
    s = ctypes.c_float()
    r = ctypes.c_float()
    lib().rxo_block_scale(x.ctypes.data, x.size, fmt, ctypes.byref(s), ctypes.byref(r))
    return s.value, r.value


def block_scale_bits(first: int, n: int, fmt: int) -> Tuple[np.ndarray, np.ndarray]:
    s = np.empty(n, dtype=np.float32)
    r = np.empty(n, dtype=np.float32)
    lib().rxo_block_scale_bits_range(first, n, fmt, s.ctypes.data, r.ctypes.data)
    return s, r


# ---- hot-path operations -------------------------------------------------

def reduce_flat(srcs: Sequence[np.ndarray], dtype: int, count: Optional[int] = None) -> np.ndarray:
    count = srcs[0].size if count is None else count
    _check(srcs, _np_of(dtype), count)
    out = np.empty(count, dtype=_np_of(dtype))
    lib().rxo_reduce_flat(_ptrs(srcs), len(srcs), count, dtype, out.ctypes.data)
    return out


def tree_chunk(count: int, nsrc: int, dtype: int, rank: int) -> Tuple[int, int]:
    lo = ctypes.c_size_t()
    hi = ctypes.c_size_t()
    lib().rxo_tree_chunk(count, nsrc, dtype, rank, ctypes.byref(lo), ctypes.byref(hi))
    return lo.value, hi.value


def reduce_scatter_chunk_bcast(srcs: Sequence[np.ndarray], dtype: int, rank: int,
                               dsts: Sequence[np.ndarray], count: Optional[int] = None) -> None:
    """Writes chunk ``rank`` of the reduction into every array of ``dsts``."""
    count = srcs[0].size if count is None else count
    _check(srcs, _np_of(dtype), count)
    _check(dsts, _np_of(dtype), count)
    assert len(dsts) == len(srcs)
    lib().rxo_reduce_scatter_chunk_bcast(_ptrs(srcs), len(srcs), count, dtype,
                                         rank, _ptrs(dsts))


def quant_fp8(srcs: Sequence[np.ndarray], src_dtype: int, fmt: int, block: int,
              count: Optional[int] = None) -> Tuple[List[np.ndarray], List[np.ndarray]]:
    count = srcs[0].size if count is None else count
    _check(srcs, _np_of(src_dtype), count)
    nb = (count + block - 1) // block
    codes = [np.empty(count, dtype=np.uint8) for _ in srcs]
    scales = [np.empty(nb, dtype=np.float32) for _ in srcs]
    lib().rxo_quant_fp8(_ptrs(srcs), len(srcs), count, src_dtype, fmt, block,
                        _ptrs(codes), _ptrs(scales))
    return codes, scales


def dequant_reduce_requant(codes: Sequence[np.ndarray], scales: Sequence[np.ndarray],
                           fmt: int, block: int, mode: int, hp_dtype: int = FP32,
                           want_hp: bool = True, count: Optional[int] = None):
    """Returns (out_codes, out_scales, out_hp); absent outputs are None."""
    count = codes[0].size if count is None else count
    _check(codes, np.uint8, count)
    nb = (count + block - 1) // block
    _check(scales, np.float32, nb)
    out_codes = out_scales = None
    cptr = sptr = None
    if mode == DRR_REQUANT:
        out_codes = np.empty(count, dtype=np.uint8)
        out_scales = np.empty(nb, dtype=np.float32)
        cptr, sptr = out_codes.ctypes.data, out_scales.ctypes.data
    out_hp = None
    hptr = None
    if mode == DRR_SUM or want_hp:
        out_hp = np.empty(count, dtype=_np_of(hp_dtype))
        hptr = out_hp.ctypes.data
    lib().rxo_dequant_reduce_requant(_ptrs(codes), _ptrs(scales), len(codes), count,
                                     fmt, block, mode, cptr, sptr, hptr, hp_dtype)
    return out_codes, out_scales, out_hp


def lp_tree_chunk(count: int, nsrc: int, block: int, rank: int) -> Tuple[int, int]:
    lo = ctypes.c_size_t()
    hi = ctypes.c_size_t()
    lib().rxo_lp_tree_chunk(count, nsrc, block, rank, ctypes.byref(lo), ctypes.byref(hi))
    return lo.value, hi.value


def lp_reduce_scatter_chunk_bcast(codes: Sequence[np.ndarray], scales: Sequence[np.ndarray],
                                  fmt: int, block: int, rank: int,
                                  dst_codes: Sequence[np.ndarray], dst_scales: Sequence[np.ndarray],
                                  out_hp: Optional[np.ndarray] = None, hp_dtype: int = FP32,
                                  count: Optional[int] = None) -> None:
    """Writes the requantized chunk `rank` into every dst_codes[j] /
    dst_scales[j] (and its dequantized values into out_hp when given)."""
    count = codes[0].size if count is None else count
    nb = (count + block - 1) // block
    _check(codes, np.uint8, count)
    _check(scales, np.float32, nb)
    _check(dst_codes, np.uint8, count)
    _check(dst_scales, np.float32, nb)
    assert len(codes) == len(scales) == len(dst_codes) == len(dst_scales)
    hptr = None
    if out_hp is not None:
        _check([out_hp], _np_of(hp_dtype), count)
        hptr = out_hp.ctypes.data
    lib().rxo_lp_reduce_scatter_chunk_bcast(_ptrs(codes), _ptrs(scales), len(codes), count,
                                            fmt, block, rank, _ptrs(dst_codes),
                                            _ptrs(dst_scales), hptr, hp_dtype)


def allreduce_local(bufs: Sequence[np.ndarray], dtype: int, algo: int, fmt: int = E4M3,
                    block: int = 128, count: Optional[int] = None) -> None:
    """In place: every array of ``bufs`` receives the allreduce result."""
    count = bufs[0].size if count is None else count
    _check(bufs, _np_of(dtype), count)
    lib().rxo_allreduce_local(_ptrs(bufs), len(bufs), count, dtype, algo, fmt, block)
