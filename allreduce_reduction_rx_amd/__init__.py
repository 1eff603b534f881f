"""Python binding of librx (``include/rx.h``): argument marshalling only.

Every function here has the name of the C entry point it calls and takes
torch tensors that live on the GPU; it checks dtype, device, contiguity and
sizes, passes ``data_ptr()`` values and the current HIP stream, and raises
``RxError`` on a non-zero status. All computation runs in librx's gfx950
kernels; there is no CPU fallback. If ``librx.so`` is missing, importing the
binding's entry points raises.

The C ABI is asynchronous (stream-ordered); these wrappers do not
synchronize.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

__all__ = [
    "RX_FP32", "RX_BF16", "RX_FP8_E4M3", "RX_FP8_E5M2", "RX_DRR_SUM",
    "RX_DRR_REQUANT", "RX_MAX_SRC", "RxError", "lib", "lib_path",
    "rx_reduce_flat", "rx_reduce_scatter_chunk_bcast", "rx_tree_chunk",
    "rx_quant_fp8", "rx_dequant_reduce_requant", "rx_status_string",
    "rx_lp_reduce_scatter_chunk_bcast", "rx_lp_tree_chunk", "rx_allreduce_local",
    "rx_allreduce_local_workspace", "rx_allreduce_local_noalloc",
    "RX_NOALLOC_SCRATCH_BYTES", "RX_ALGO_AUTO", "RX_ALGO_FLAT", "RX_ALGO_TREE",
    "RX_ALGO_LOWPREC", "EXPORTED_SYMBOLS",
]

RX_FP32, RX_BF16, RX_FP8_E4M3, RX_FP8_E5M2 = 0, 1, 2, 3
RX_DRR_SUM, RX_DRR_REQUANT = 0, 1
RX_ALGO_AUTO, RX_ALGO_FLAT, RX_ALGO_TREE, RX_ALGO_LOWPREC = 0, 1, 2, 3
RX_MAX_SRC = 16
RX_NOALLOC_SCRATCH_BYTES = 64 << 20
RX_ERR_SCRATCH = 6

EXPORTED_SYMBOLS = (
    "rx_reduce_flat", "rx_reduce_scatter_chunk_bcast", "rx_tree_chunk",
    "rx_quant_fp8", "rx_dequant_reduce_requant", "rx_status_string",
    "rx_lp_reduce_scatter_chunk_bcast", "rx_lp_tree_chunk", "rx_allreduce_local",
    "rx_allreduce_local_workspace", "rx_allreduce_local_noalloc", "rxtest_block_scale_bits", "rxtest_fp8_encode_bits", "rxtest_fp8_decode", "rxtest_bf16_round_bits",
    "rxtest_group_max", "rxtest_stream", "rxtest_stream_sink_bytes", "rxtest_stream_mixed",
    "rxtest_copy_streams",
)

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(_HERE, "librx.so")


class RxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {rx_status_string(status)} ({status})")


_lib = None
_P = ctypes.c_void_p
_PP = ctypes.POINTER(ctypes.c_void_p)
_SZ = ctypes.c_size_t
_I = ctypes.c_int


def lib() -> ctypes.CDLL:
    """Loads librx.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with __graft_entry__.build()")
        # torch ships its own HIP runtime under the same soname as the system
        # one librx is linked against. With torch loaded first, the loader
        # resolves librx to that runtime: one HIP runtime in the process.
        # Loading librx first would bind it to the system runtime, and torch
        # would then map its bundled copy beside it (two HIP runtimes, whose
        # device memory, streams and modules the other does not know).
        import torch  # noqa: F401
        L = ctypes.CDLL(path)
        sig = {
            "rx_reduce_flat": [_PP, _I, _SZ, _I, _P, _P],
            "rx_reduce_scatter_chunk_bcast": [_PP, _I, _SZ, _I, _I, _PP, _P],
            "rx_tree_chunk": [_SZ, _I, _I, _I, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)],
            "rx_quant_fp8": [_PP, _I, _SZ, _I, _I, _I, _PP, _PP, _P],
            "rx_dequant_reduce_requant": [_PP, _PP, _I, _SZ, _I, _I, _I, _P, _P, _P, _I, _P],
            "rx_lp_reduce_scatter_chunk_bcast": [_PP, _PP, _I, _SZ, _I, _I, _I, _PP, _PP, _P,
                                                 _I, _P],
            "rx_lp_tree_chunk": [_SZ, _I, _I, _I, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)],
            "rx_allreduce_local": [_PP, _I, _SZ, _I, _I, _I, _I, _P, _SZ, _P],
            "rx_allreduce_local_noalloc": [_PP, _I, _SZ, _I, _I, _I, _I, _P],
            "rxtest_fp8_encode_bits": [ctypes.c_uint32, _SZ, _I, _P, _P],
            "rxtest_block_scale_bits": [ctypes.c_uint32, _SZ, _I, _P, _P, _P],
            "rxtest_fp8_decode": [_P, _SZ, _I, _P, _P],
            "rxtest_bf16_round_bits": [ctypes.c_uint32, _SZ, _P, _P],
            "rxtest_group_max": [_P, _SZ, _I, _P, _P],
            "rxtest_stream": [_I, _P, _P, _SZ, _I, _I, _P],
            "rxtest_stream_mixed": [_I, _PP, _I, _P, _SZ, _I, _I, _I, _P],
            "rxtest_copy_streams": [_PP, _PP, _I, _SZ, _SZ, _I, _I, _P],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.rxtest_stream_sink_bytes.argtypes = [_I]
        L.rxtest_stream_sink_bytes.restype = ctypes.c_size_t
        L.rx_allreduce_local_workspace.argtypes = [_I, _SZ, _I]
        L.rx_allreduce_local_workspace.restype = ctypes.c_size_t
        L.rx_status_string.argtypes = [_I]
        L.rx_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def rx_status_string(status: int) -> str:
    return lib().rx_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise RxError(status, where)


def _ptr_array(values: Sequence[int]):
    return (ctypes.c_void_p * max(1, len(values)))(*values)


def _stream(stream) -> int:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _rx_dtype(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return RX_FP32
    if t.dtype == torch.bfloat16:
        return RX_BF16
    raise TypeError(f"unsupported tensor dtype {t.dtype} (float32 or bfloat16)")


def _gpu(t, name: str) -> None:
    import torch
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, the current device is "
                         f"cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _fp8_code(fmt) -> int:
    if isinstance(fmt, str):
        return {"e4m3": RX_FP8_E4M3, "e5m2": RX_FP8_E5M2}[fmt.lower()]
    return int(fmt)


def rx_reduce_flat(srcs: Sequence, dst, count: Optional[int] = None, stream=None) -> None:
    """dst[i] = FP32 left fold of srcs[0][i] .. srcs[n-1][i], cast to dst's dtype."""
    count = dst.numel() if count is None else count
    dt = _rx_dtype(dst)
    for k, s in enumerate(srcs):
        _gpu(s, f"srcs[{k}]")
        if s.dtype != dst.dtype or s.numel() < count:
            raise ValueError(f"srcs[{k}] must be {dst.dtype} with >= {count} elements")
    _gpu(dst, "dst")
    if dst.numel() < count:
        raise ValueError("dst too small")
    arr = _ptr_array([s.data_ptr() for s in srcs])
    _check(lib().rx_reduce_flat(arr, len(srcs), count, dt, dst.data_ptr(), _stream(stream)),
           "rx_reduce_flat")


def rx_tree_chunk(count: int, nsrc: int, dtype: int, rank: int) -> Tuple[int, int]:
    lo, hi = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().rx_tree_chunk(count, nsrc, dtype, rank, ctypes.byref(lo), ctypes.byref(hi)),
           "rx_tree_chunk")
    return lo.value, hi.value


def rx_reduce_scatter_chunk_bcast(srcs: Sequence, rank: int, dsts: Sequence,
                                  count: Optional[int] = None, stream=None) -> None:
    """Reduce chunk `rank` across srcs and write it into every dsts[j]."""
    count = srcs[0].numel() if count is None else count
    dt = _rx_dtype(srcs[0])
    if len(dsts) != len(srcs):
        raise ValueError("need one destination per source")
    for k, t in enumerate(list(srcs) + list(dsts)):
        _gpu(t, f"buffer {k}")
        if t.dtype != srcs[0].dtype or t.numel() < count:
            raise ValueError(f"buffer {k} must be {srcs[0].dtype} with >= {count} elements")
    sa = _ptr_array([s.data_ptr() for s in srcs])
    da = _ptr_array([d.data_ptr() for d in dsts])
    _check(lib().rx_reduce_scatter_chunk_bcast(sa, len(srcs), count, dt, rank, da, _stream(stream)),
           "rx_reduce_scatter_chunk_bcast")


def rx_quant_fp8(srcs: Sequence, fmt, block: int, codes: Sequence, scales: Sequence,
                 count: Optional[int] = None, stream=None) -> None:
    """codes[j] (uint8, count) and scales[j] (float32, ceil(count/block)) from srcs[j]."""
    import torch
    count = srcs[0].numel() if count is None else count
    dt = _rx_dtype(srcs[0])
    nb = -(-count // block) if block > 0 else 0
    if not (len(srcs) == len(codes) == len(scales)):
        raise ValueError("need one code and one scale buffer per source")
    for k, s in enumerate(srcs):
        _gpu(s, f"srcs[{k}]")
        if s.dtype != srcs[0].dtype or s.numel() < count:
            raise ValueError(f"srcs[{k}] must be {srcs[0].dtype} with >= {count} elements")
    for k, (c, sc) in enumerate(zip(codes, scales)):
        _gpu(c, f"codes[{k}]")
        _gpu(sc, f"scales[{k}]")
        if c.dtype != torch.uint8 or c.numel() < count:
            raise ValueError(f"codes[{k}] must be uint8 with >= {count} elements")
        if sc.dtype != torch.float32 or sc.numel() < nb:
            raise ValueError(f"scales[{k}] must be float32 with >= {nb} elements")
    sa = _ptr_array([s.data_ptr() for s in srcs])
    ca = _ptr_array([c.data_ptr() for c in codes])
    qa = _ptr_array([s.data_ptr() for s in scales])
    _check(lib().rx_quant_fp8(sa, len(srcs), count, dt, _fp8_code(fmt), block, ca, qa,
                              _stream(stream)), "rx_quant_fp8")


def rx_dequant_reduce_requant(codes: Sequence, scales: Sequence, fmt, block: int, mode: int,
                              out_codes=None, out_scales=None, out_hp=None,
                              count: Optional[int] = None, stream=None) -> None:
    """Dequantize + FP32 sum; SUM writes out_hp, REQUANT writes out_codes /
    out_scales (and out_hp = dequant(requant(sum)) when given)."""
    import torch
    count = codes[0].numel() if count is None else count
    nb = -(-count // block) if block > 0 else 0
    if len(codes) != len(scales):
        raise ValueError("need one scale buffer per code buffer")
    for k, (c, sc) in enumerate(zip(codes, scales)):
        _gpu(c, f"codes[{k}]")
        _gpu(sc, f"scales[{k}]")
        if c.dtype != torch.uint8 or c.numel() < count:
            raise ValueError(f"codes[{k}] must be uint8 with >= {count} elements")
        if sc.dtype != torch.float32 or sc.numel() < nb:
            raise ValueError(f"scales[{k}] must be float32 with >= {nb} elements")
    hp_dt = RX_FP32
    if out_hp is not None:
        _gpu(out_hp, "out_hp")
        hp_dt = _rx_dtype(out_hp)
        if out_hp.numel() < count:
            raise ValueError("out_hp too small")
    if out_codes is not None:
        _gpu(out_codes, "out_codes")
        if out_codes.dtype != torch.uint8 or out_codes.numel() < count:
            raise ValueError("out_codes must be uint8 with >= count elements")
    if out_scales is not None:
        _gpu(out_scales, "out_scales")
        if out_scales.dtype != torch.float32 or out_scales.numel() < nb:
            raise ValueError("out_scales must be float32 with >= ceil(count/block) elements")
    ca = _ptr_array([c.data_ptr() for c in codes])
    qa = _ptr_array([s.data_ptr() for s in scales])
    ptr = lambda t: None if t is None else t.data_ptr()
    _check(lib().rx_dequant_reduce_requant(ca, qa, len(codes), count, _fp8_code(fmt), block,
                                           mode, ptr(out_codes), ptr(out_scales), ptr(out_hp),
                                           hp_dt, _stream(stream)),
           "rx_dequant_reduce_requant")


def rx_lp_tree_chunk(count: int, nsrc: int, block: int, rank: int) -> Tuple[int, int]:
    lo, hi = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().rx_lp_tree_chunk(count, nsrc, block, rank, ctypes.byref(lo), ctypes.byref(hi)),
           "rx_lp_tree_chunk")
    return lo.value, hi.value


def rx_lp_reduce_scatter_chunk_bcast(codes: Sequence, scales: Sequence, fmt, block: int,
                                     rank: int, dst_codes: Sequence, dst_scales: Sequence,
                                     out_hp=None, count: Optional[int] = None,
                                     stream=None) -> None:
    """Requantized chunk `rank` of the FP32 sum of the dequantized inputs,
    pushed into every dst_codes[j] / dst_scales[j] (and out_hp when given)."""
    import torch
    count = codes[0].numel() if count is None else count
    nb = -(-count // block) if block > 0 else 0
    n = len(codes)
    if not (len(scales) == len(dst_codes) == len(dst_scales) == n):
        raise ValueError("need one scale, destination-code and destination-scale buffer per rank")
    for k in range(n):
        for name, t, dt, need in (("codes", codes[k], torch.uint8, count),
                                  ("scales", scales[k], torch.float32, nb),
                                  ("dst_codes", dst_codes[k], torch.uint8, count),
                                  ("dst_scales", dst_scales[k], torch.float32, nb)):
            _gpu(t, f"{name}[{k}]")
            if t.dtype != dt or t.numel() < need:
                raise ValueError(f"{name}[{k}] must be {dt} with >= {need} elements")
    hp_dt = RX_FP32
    if out_hp is not None:
        _gpu(out_hp, "out_hp")
        hp_dt = _rx_dtype(out_hp)
        if out_hp.numel() < count:
            raise ValueError("out_hp too small")
    arr = lambda ts: _ptr_array([t.data_ptr() for t in ts])
    _check(lib().rx_lp_reduce_scatter_chunk_bcast(
        arr(codes), arr(scales), n, count, _fp8_code(fmt), block, rank, arr(dst_codes),
        arr(dst_scales), None if out_hp is None else out_hp.data_ptr(), hp_dt, _stream(stream)),
        "rx_lp_reduce_scatter_chunk_bcast")


def rx_allreduce_local_workspace(nsrc: int, count: int, block: int) -> int:
    """Workspace bytes rx_allreduce_local needs for the low-precision algorithm."""
    return int(lib().rx_allreduce_local_workspace(nsrc, count, block))


def rx_allreduce_local(bufs: Sequence, algo: int = RX_ALGO_AUTO, fmt="e4m3", block: int = 128,
                       workspace=None, count: Optional[int] = None, stream=None) -> None:
    """In-place SUM allreduce of the rank buffers `bufs` (all on this GPU):
    afterwards every buffer holds the result. `workspace` (a uint8 GPU tensor
    of rx_allreduce_local_workspace() bytes) is needed by the low-precision
    algorithm only."""
    import torch
    count = bufs[0].numel() if count is None else count
    dt = _rx_dtype(bufs[0])
    for k, t in enumerate(bufs):
        _gpu(t, f"bufs[{k}]")
        if t.dtype != bufs[0].dtype or t.numel() < count:
            raise ValueError(f"bufs[{k}] must be {bufs[0].dtype} with >= {count} elements")
    wptr, wbytes = None, 0
    if workspace is not None:
        _gpu(workspace, "workspace")
        if workspace.dtype != torch.uint8:
            raise ValueError("workspace must be a uint8 tensor")
        wptr, wbytes = workspace.data_ptr(), workspace.numel()
    _check(lib().rx_allreduce_local(_ptr_array([t.data_ptr() for t in bufs]), len(bufs), count,
                                    dt, int(algo), _fp8_code(fmt), block, wptr, wbytes,
                                    _stream(stream)), "rx_allreduce_local")


def rx_allreduce_local_noalloc(bufs: Sequence, algo: int = RX_ALGO_AUTO, fmt="e4m3",
                               block: int = 128, count: Optional[int] = None,
                               stream=None) -> None:
    """rx_allreduce_local without a workspace: the low-precision algorithm
    uses the library's per-device scratch (RX_NOALLOC_SCRATCH_BYTES), so
    nothing is allocated; calls that overlap on one device race on it."""
    count = bufs[0].numel() if count is None else count
    dt = _rx_dtype(bufs[0])
    for k, t in enumerate(bufs):
        _gpu(t, f"bufs[{k}]")
        if t.dtype != bufs[0].dtype or t.numel() < count:
            raise ValueError(f"bufs[{k}] must be {bufs[0].dtype} with >= {count} elements")
    _check(lib().rx_allreduce_local_noalloc(_ptr_array([t.data_ptr() for t in bufs]), len(bufs),
                                            count, dt, int(algo), _fp8_code(fmt), block,
                                            _stream(stream)), "rx_allreduce_local_noalloc")


# ---- test hooks (rx_testhooks.h) -------------------------------------------

def _hook_buf(t, name: str, nbytes: int) -> None:
    _gpu(t, name)
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} must hold {nbytes} bytes")


def rxtest_fp8_encode_bits(first: int, n: int, fmt, out, stream=None) -> None:
    _hook_buf(out, "out", n)
    _check(lib().rxtest_fp8_encode_bits(first, n, _fp8_code(fmt), out.data_ptr(), _stream(stream)),
           "rxtest_fp8_encode_bits")


def rxtest_block_scale_bits(first: int, n: int, fmt, s, r, stream=None) -> None:
    _hook_buf(s, "s", 4 * n)
    _hook_buf(r, "r", 4 * n)
    _check(lib().rxtest_block_scale_bits(first, n, _fp8_code(fmt), s.data_ptr(), r.data_ptr(),
                                         _stream(stream)), "rxtest_block_scale_bits")


def rxtest_fp8_decode(codes, fmt, out, stream=None) -> None:
    _hook_buf(codes, "codes", codes.numel())
    _hook_buf(out, "out", 4 * codes.numel())
    _check(lib().rxtest_fp8_decode(codes.data_ptr(), codes.numel(), _fp8_code(fmt),
                                   out.data_ptr(), _stream(stream)), "rxtest_fp8_decode")


def rxtest_bf16_round_bits(first: int, n: int, out, stream=None) -> None:
    _hook_buf(out, "out", 2 * n)
    _check(lib().rxtest_bf16_round_bits(first, n, out.data_ptr(), _stream(stream)),
           "rxtest_bf16_round_bits")


def rxtest_group_max(values, g: int, out, stream=None) -> None:
    nw = values.numel() // 64
    _hook_buf(values, "values", 4 * 64 * nw)
    _hook_buf(out, "out", 4 * 64 * nw)
    _check(lib().rxtest_group_max(values.data_ptr(), nw, g, out.data_ptr(),
                                  _stream(stream)), "rxtest_group_max")


RXTEST_READ, RXTEST_WRITE, RXTEST_COPY, RXTEST_EMPTY = 0, 1, 2, 3


def rxtest_stream_sink_bytes(wgs_per_cu: int) -> int:
    return int(lib().rxtest_stream_sink_bytes(wgs_per_cu))


def rxtest_stream(kind: int, src, dst, nbytes: int, wgs_per_cu: int = 1, nontemporal: bool = False,
                  stream=None) -> None:
    """Streaming ceiling kernel (read / write / copy / empty) over nbytes; for
    a read, dst is the per-wave XOR sink of rxtest_stream_sink_bytes(wgs_per_cu)."""
    def size(t):
        return t.numel() * t.element_size()
    for name, t in (("src", src), ("dst", dst)):
        if t is not None:
            _gpu(t, name)
    if kind in (RXTEST_READ, RXTEST_COPY) and (src is None or size(src) < nbytes):
        raise ValueError("src must hold nbytes")
    if kind in (RXTEST_WRITE, RXTEST_COPY) and (dst is None or size(dst) < nbytes):
        raise ValueError("dst must hold nbytes")
    if kind == RXTEST_READ and (dst is None or size(dst) < rxtest_stream_sink_bytes(wgs_per_cu)):
        raise ValueError("dst must hold rxtest_stream_sink_bytes(wgs_per_cu) bytes")
    _check(lib().rxtest_stream(kind, src.data_ptr() if src is not None else None,
                               dst.data_ptr() if dst is not None else None,
                               nbytes, wgs_per_cu, int(bool(nontemporal)), _stream(stream)),
           "rxtest_stream")


RXTEST_MIXED_REDUCE, RXTEST_MIXED_NARROW2, RXTEST_MIXED_NARROW4 = 0, 1, 2


def rxtest_stream_mixed(kind: int, srcs: Sequence, dst, src_bytes: int, wgs_per_cu: int = 1,
                        nontemporal: bool = False, prefetch: bool = False, stream=None) -> None:
    """Mixed read/write ceiling kernel: reduce (len(srcs) : 1, dst = XOR of
    the sources) or narrow (one source, dst of src_bytes / 2 or / 4)."""
    def size(t):
        return t.numel() * t.element_size()
    for k, t in enumerate(srcs):
        _gpu(t, f"srcs[{k}]")
        if size(t) < src_bytes:
            raise ValueError(f"srcs[{k}] must hold src_bytes")
    _gpu(dst, "dst")
    out = src_bytes // {RXTEST_MIXED_REDUCE: 1, RXTEST_MIXED_NARROW2: 2,
                        RXTEST_MIXED_NARROW4: 4}.get(kind, 1)
    if size(dst) < out:
        raise ValueError("dst too small")
    _check(lib().rxtest_stream_mixed(kind, _ptr_array([t.data_ptr() for t in srcs]), len(srcs),
                                     dst.data_ptr(), src_bytes, wgs_per_cu,
                                     int(bool(nontemporal)), int(bool(prefetch)), _stream(stream)),
           "rxtest_stream_mixed")


def rxtest_copy_streams(srcs: Sequence, dsts: Sequence, offset_bytes: int, nbytes: int,
                        lanes: int = 1, wg: int = 64, stream=None) -> None:
    """The tree step's memory pattern without its arithmetic: bytes
    [offset_bytes, offset_bytes + nbytes) of srcs[j] copied into dsts[j]."""
    def size(t):
        return t.numel() * t.element_size()
    if len(srcs) != len(dsts):
        raise ValueError("srcs and dsts must have the same length")
    for name, ts in (("srcs", srcs), ("dsts", dsts)):
        for k, t in enumerate(ts):
            _gpu(t, f"{name}[{k}]")
            if size(t) < offset_bytes + nbytes:
                raise ValueError(f"{name}[{k}] must hold offset_bytes + nbytes")
    _check(lib().rxtest_copy_streams(_ptr_array([t.data_ptr() for t in srcs]),
                                     _ptr_array([t.data_ptr() for t in dsts]), len(srcs),
                                     offset_bytes, nbytes, lanes, wg, _stream(stream)),
           "rxtest_copy_streams")
