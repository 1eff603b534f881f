"""Host-side checks of the C ABI that need no GPU: the library loads, it
exports every function its headers declare, and argument validation returns
the documented status before any HIP call (no kernel is launched: every
call here fails validation or has count == 0). Device pointers are fake
addresses that are never dereferenced on the host."""
import ctypes
import os
import re

import pytest

import allreduce_reduction_rx_amd as rx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, ARG, DTYPE, ALIGN, HIP, SCRATCH = 0, 1, 2, 3, 4, 5, 6
FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced


def declared_functions():
    names = set()
    for h in os.listdir(os.path.join(ROOT, "include")):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            names |= set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(rx\w*)\s*\(", text, re.M))
    return names


def test_headers_declare_the_four_entry_points():
    names = declared_functions()
    for n in ("rx_reduce_flat", "rx_reduce_scatter_chunk_bcast", "rx_quant_fp8",
              "rx_dequant_reduce_requant"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = rx.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(declared_functions()) <= set(rx.EXPORTED_SYMBOLS)


def ptrs(*vals):
    return (ctypes.c_void_p * max(1, len(vals)))(*vals)


def test_status_strings():
    for s in range(7):
        assert rx.rx_status_string(s).startswith("RX_")


def test_reduce_flat_validation():
    L = rx.lib()
    f = L.rx_reduce_flat
    src = ptrs(FAKE, FAKE + 4096)
    assert f(None, 2, 10, rx.RX_FP32, FAKE, None) == NULL
    assert f(src, 2, 10, rx.RX_FP32, None, None) == NULL
    assert f(src, 0, 10, rx.RX_FP32, FAKE, None) == ARG
    assert f(src, 17, 10, rx.RX_FP32, FAKE, None) == ARG
    assert f(src, 2, 10, rx.RX_FP8_E4M3, FAKE, None) == DTYPE
    assert f(src, 2, 10, 9, FAKE, None) == DTYPE
    assert f(ptrs(FAKE, 0), 2, 10, rx.RX_FP32, FAKE, None) == NULL
    assert f(ptrs(FAKE, FAKE + 8), 2, 10, rx.RX_FP32, FAKE, None) == ALIGN
    assert f(src, 2, 10, rx.RX_FP32, FAKE + 4, None) == ALIGN
    assert f(src, 2, 0, rx.RX_BF16, FAKE, None) == OK  # nothing to do, no launch
    assert f(src, 2, (1 << 38) + 1, rx.RX_FP32, FAKE, None) == ARG


def test_tree_validation_and_chunks():
    L = rx.lib()
    f = L.rx_reduce_scatter_chunk_bcast
    src, dst = ptrs(FAKE, FAKE + 4096), ptrs(FAKE + 8192, FAKE + 12288)
    assert f(src, 2, 10, rx.RX_FP32, 2, dst, None) == ARG
    assert f(src, 2, 10, rx.RX_FP32, -1, dst, None) == ARG
    assert f(src, 2, 10, rx.RX_FP32, 0, None, None) == NULL
    assert f(src, 2, 10, rx.RX_FP32, 0, ptrs(FAKE + 8192, FAKE + 2), None) == ALIGN
    assert f(src, 2, 0, rx.RX_FP32, 1, dst, None) == OK
    # chunk bounds of the 4 MiB BF16 tree message, 8 ranks: 262,144 each
    for k in range(8):
        assert rx.rx_tree_chunk(2_097_152, 8, rx.RX_BF16, k) == (k * 262_144, (k + 1) * 262_144)
    # ragged: 10 FP32 over 4 ranks -> chunks of 4: [0,4) [4,8) [8,10) [10,10)
    assert [rx.rx_tree_chunk(10, 4, rx.RX_FP32, k) for k in range(4)] == [(0, 4), (4, 8), (8, 10), (10, 10)]
    # an empty chunk launches nothing
    assert f(src, 2, 3, rx.RX_FP32, 1, dst, None) == OK


def test_quant_validation():
    L = rx.lib()
    f = L.rx_quant_fp8
    src, codes, sc = ptrs(FAKE), ptrs(FAKE + 4096), ptrs(FAKE + 8192)
    assert f(src, 1, 100, rx.RX_FP32, rx.RX_FP8_E4M3, 128, None, sc, None) == NULL
    assert f(src, 1, 100, rx.RX_FP32, rx.RX_FP8_E4M3, 100, codes, sc, None) == ARG
    assert f(src, 1, 100, rx.RX_FP32, rx.RX_FP8_E4M3, 16, codes, sc, None) == ARG
    assert f(src, 1, 100, rx.RX_FP32, rx.RX_FP8_E4M3, 2048, codes, sc, None) == ARG
    assert f(src, 1, 100, rx.RX_FP8_E5M2, rx.RX_FP8_E4M3, 128, codes, sc, None) == DTYPE
    assert f(src, 1, 100, rx.RX_FP32, rx.RX_BF16, 128, codes, sc, None) == DTYPE
    assert f(src, 1, 100, rx.RX_FP32, rx.RX_FP8_E4M3, 128, ptrs(FAKE + 1), sc, None) == ALIGN
    assert f(src, 1, 100, rx.RX_FP32, rx.RX_FP8_E4M3, 128, codes, ptrs(FAKE + 2), None) == ALIGN
    assert f(src, 1, 0, rx.RX_BF16, rx.RX_FP8_E5M2, 256, codes, sc, None) == OK
    src16 = ptrs(*([FAKE] * 16))
    c16, s16 = ptrs(*([FAKE + 4096] * 16)), ptrs(*([FAKE + 8192] * 16))
    assert f(src16, 16, (1 << 36), rx.RX_FP32, rx.RX_FP8_E4M3, 128, c16, s16, None) == ARG


def test_drr_validation():
    L = rx.lib()
    f = L.rx_dequant_reduce_requant
    c, s = ptrs(FAKE, FAKE + 4096), ptrs(FAKE + 8192, FAKE + 12288)
    E4, SUM, REQ = rx.RX_FP8_E4M3, rx.RX_DRR_SUM, rx.RX_DRR_REQUANT
    out = FAKE + 65536
    assert f(None, s, 2, 10, E4, 128, SUM, None, None, out, rx.RX_FP32, None) == NULL
    assert f(c, s, 2, 10, E4, 128, 7, None, None, out, rx.RX_FP32, None) == ARG
    assert f(c, s, 2, 10, E4, 128, SUM, None, None, None, rx.RX_FP32, None) == NULL
    assert f(c, s, 2, 10, E4, 128, SUM, out, None, out, rx.RX_FP32, None) == ARG
    assert f(c, s, 2, 10, E4, 128, REQ, None, out, None, rx.RX_FP32, None) == NULL
    assert f(c, s, 2, 10, rx.RX_BF16, 128, SUM, None, None, out, rx.RX_FP32, None) == DTYPE
    assert f(c, s, 2, 10, E4, 128, SUM, None, None, out, rx.RX_FP8_E5M2, None) == DTYPE
    assert f(c, s, 2, 10, E4, 48, SUM, None, None, out, rx.RX_FP32, None) == ARG
    assert f(c, s, 2, 10, E4, 128, REQ, out + 3, out, None, rx.RX_FP32, None) == ALIGN
    assert f(c, s, 2, 10, E4, 128, REQ, out, out + 1, None, rx.RX_FP32, None) == ALIGN
    assert f(c, s, 2, 10, E4, 128, SUM, None, None, out + 8, rx.RX_BF16, None) == ALIGN
    assert f(c, ptrs(FAKE, FAKE + 3), 2, 10, E4, 128, SUM, None, None, out, rx.RX_FP32, None) == ALIGN
    assert f(c, s, 2, 0, E4, 128, REQ, out, out, None, rx.RX_FP32, None) == OK


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(8)
    with pytest.raises(ValueError):
        rx.rx_reduce_flat([x], x)


def test_lp_tree_validation_and_chunks():
    L = rx.lib()
    f = L.rx_lp_reduce_scatter_chunk_bcast
    c, s = ptrs(FAKE, FAKE + 4096), ptrs(FAKE + 8192, FAKE + 12288)
    dc, ds = ptrs(FAKE + 16384, FAKE + 20480), ptrs(FAKE + 24576, FAKE + 28672)
    E4 = rx.RX_FP8_E4M3
    assert f(None, s, 2, 1000, E4, 128, 0, dc, ds, None, rx.RX_FP32, None) == NULL
    assert f(c, s, 2, 1000, E4, 128, 0, None, ds, None, rx.RX_FP32, None) == NULL
    assert f(c, s, 2, 1000, E4, 128, 2, dc, ds, None, rx.RX_FP32, None) == ARG
    assert f(c, s, 2, 1000, E4, 96, 0, dc, ds, None, rx.RX_FP32, None) == ARG
    assert f(c, s, 2, 1000, rx.RX_FP32, 128, 0, dc, ds, None, rx.RX_FP32, None) == DTYPE
    assert f(c, s, 2, 1000, E4, 128, 0, dc, ds, FAKE, rx.RX_FP8_E5M2, None) == DTYPE
    assert f(c, s, 2, 1000, E4, 128, 0, ptrs(FAKE + 16384, FAKE + 8), ds, None, rx.RX_FP32, None) == ALIGN
    assert f(c, s, 2, 1000, E4, 128, 0, dc, ptrs(FAKE, FAKE + 1), None, rx.RX_FP32, None) == ALIGN
    assert f(c, s, 2, 1000, E4, 128, 0, dc, ds, FAKE + 4, rx.RX_BF16, None) == ALIGN
    assert f(c, s, 2, 0, E4, 128, 1, dc, ds, None, rx.RX_FP32, None) == OK
    # 8 ranks over the 64 MiB FP32 low-precision message, blocks of 128
    for k in range(8):
        assert rx.rx_lp_tree_chunk(16_777_216, 8, 128, k) == (k * 2_097_152, (k + 1) * 2_097_152)
    assert [rx.rx_lp_tree_chunk(1000, 3, 128, k) for k in range(3)] == [(0, 384), (384, 768), (768, 1000)]
    # an empty chunk launches nothing
    assert f(c, s, 2, 100, E4, 128, 1, dc, ds, None, rx.RX_FP32, None) == OK


def test_allreduce_local_validation():
    L = rx.lib()
    f = L.rx_allreduce_local
    bufs = ptrs(FAKE, FAKE + 4096)
    ws = FAKE + (1 << 20)
    F32, E4 = rx.RX_FP32, rx.RX_FP8_E4M3
    FLAT, LP, AUTO = rx.RX_ALGO_FLAT, rx.RX_ALGO_LOWPREC, rx.RX_ALGO_AUTO
    need = rx.rx_allreduce_local_workspace(2, 1000, 128)
    assert need == 2 * (1024 + 256)
    assert rx.rx_allreduce_local_workspace(0, 1000, 128) == 0
    assert rx.rx_allreduce_local_workspace(2, 1000, 100) == 0
    assert f(None, 2, 1000, F32, FLAT, E4, 128, None, 0, None) == NULL
    assert f(bufs, 0, 1000, F32, FLAT, E4, 128, None, 0, None) == ARG
    assert f(bufs, 2, 1000, F32, 9, E4, 128, None, 0, None) == ARG
    assert f(bufs, 2, 1000, rx.RX_FP8_E5M2, FLAT, E4, 128, None, 0, None) == DTYPE
    assert f(ptrs(FAKE, FAKE + 2), 2, 1000, F32, FLAT, E4, 128, None, 0, None) == ALIGN
    assert f(bufs, 2, 1000, F32, LP, E4, 128, None, 0, None) == NULL
    assert f(bufs, 2, 1000, F32, LP, E4, 128, ws, need - 1, None) == ARG
    assert f(bufs, 2, 1000, F32, LP, E4, 128, ws + 16, need, None) == ALIGN
    assert f(bufs, 2, 1000, F32, LP, E4, 96, ws, need, None) == ARG
    assert f(bufs, 2, 1000, F32, LP, rx.RX_BF16, 128, ws, need, None) == DTYPE
    # the quantizer's 32-bit tile indices bound count * nsrc (checked first)
    big = ptrs(*[FAKE + 4096 * j for j in range(16)])
    assert f(big, 16, 1 << 36, F32, LP, E4, 128, ws, 1 << 62, None) == ARG
    # nothing to do: no launch
    assert f(bufs, 2, 0, F32, LP, E4, 128, ws, need, None) == OK
    assert f(bufs, 2, 0, F32, AUTO, E4, 128, None, 0, None) == OK


def test_allreduce_local_noalloc_validation():
    """The allocation-free variant validates like rx_allreduce_local and
    rejects a low-precision call whose codes and scales exceed the library's
    scratch with RX_ERR_SCRATCH, before any HIP call (so before the scratch
    address lookup, which needs a device)."""
    L = rx.lib()
    f = L.rx_allreduce_local_noalloc
    bufs = ptrs(*[FAKE + (1 << 26) * j for j in range(8)])
    F32, BF, E4, E5 = rx.RX_FP32, rx.RX_BF16, rx.RX_FP8_E4M3, rx.RX_FP8_E5M2
    FLAT, LP = rx.RX_ALGO_FLAT, rx.RX_ALGO_LOWPREC
    cap = rx.RX_NOALLOC_SCRATCH_BYTES
    assert cap == 64 << 20
    assert f(None, 8, 1000, F32, FLAT, E4, 128, None) == NULL
    assert f(bufs, 0, 1000, F32, FLAT, E4, 128, None) == ARG
    assert f(bufs, 8, 1000, F32, 9, E4, 128, None) == ARG
    assert f(bufs, 8, 1000, E5, FLAT, E4, 128, None) == DTYPE
    assert f(ptrs(FAKE, FAKE + 2), 2, 1000, F32, FLAT, E4, 128, None) == ALIGN
    assert f(bufs, 8, 1000, F32, LP, E4, 96, None) == ARG
    assert f(bufs, 8, 1000, F32, LP, BF, 128, None) == DTYPE
    # largest two-pass low-precision count that fits (blocks of 1024 are
    # beyond the one-pass limit), and the next one
    fit = 8_355_840
    assert rx.rx_allreduce_local_workspace(8, fit, 1024) <= cap
    assert rx.rx_allreduce_local_workspace(8, fit + 1, 1024) > cap
    assert f(bufs, 8, fit + 1, F32, LP, E4, 1024, None) == SCRATCH
    assert f(bufs, 8, fit + 1, F32, LP, E4, 512, None) == SCRATCH
    assert f(bufs, 8, 8 << 20, BF, LP, E5, 1024, None) == SCRATCH   # 8 x 16 MiB BF16
    assert "scratch" in rx.rx_status_string(SCRATCH)


def test_one_hip_runtime_per_process():
    """The binding loads torch before librx, so librx binds to the HIP
    runtime torch brings (same soname as the system one): a process that
    loads the library through the binding maps exactly one HIP runtime, even
    when the binding loads it before any torch import."""
    import subprocess
    import sys
    code = ("import allreduce_reduction_rx_amd as rx\n"
            "rx.lib()\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "print(sorted({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    libs = eval(r.stdout.strip().splitlines()[-1])
    assert len(libs) == 1, libs


def test_source_hash_does_not_depend_on_the_checkout_path(tmp_path):
    """A checkout at another path (the GPU machine's) with the same sources and
    stamps is not stale, so the tests never rebuild there."""
    import shutil
    import subprocess
    import sys
    for d in ("allreduce_reduction_rx_amd", "include", "oracle", "rxgen"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copy(os.path.join(ROOT, "__graft_entry__.py"), tmp_path)
    here = subprocess.run([sys.executable, "-c", "import __graft_entry__ as g; print(g.stale())"],
                          capture_output=True, text=True, cwd=ROOT, timeout=120)
    there = subprocess.run([sys.executable, "-c", "import __graft_entry__ as g; print(g.stale())"],
                           capture_output=True, text=True, cwd=str(tmp_path), timeout=120)
    assert here.stdout.strip() == "[]", here.stdout + here.stderr
    assert there.stdout.strip() == "[]", there.stdout + there.stderr


def test_stream_ceiling_validation():
    L = rx.lib()
    f = L.rxtest_stream
    assert f(4, FAKE, FAKE, 1024, 1, 0, None) == ARG        # kind
    assert f(-1, FAKE, FAKE, 1024, 1, 0, None) == ARG
    assert f(0, FAKE, FAKE, 1024, 0, 0, None) == ARG        # workgroups per CU
    assert f(0, FAKE, FAKE, 1024, 9, 0, None) == ARG
    assert f(0, None, FAKE, 1024, 1, 0, None) == NULL       # read needs src
    assert f(2, FAKE, None, 1024, 1, 0, None) == NULL
    assert f(2, FAKE, FAKE, 1000, 1, 0, None) == ALIGN      # bytes % 16
    assert f(2, FAKE + 8, FAKE, 1024, 1, 0, None) == ALIGN
    assert f(1, None, FAKE + 4, 1024, 1, 0, None) == ALIGN
    assert f(1, None, FAKE, 0, 1, 0, None) == OK            # nothing to do
    assert L.rxtest_stream_sink_bytes(0) == 0
    assert L.rxtest_stream_sink_bytes(9) == 0
    m = L.rxtest_stream_mixed
    two = ptrs(FAKE, FAKE + 4096)
    assert m(3, two, 2, FAKE, 1024, 1, 0, 0, None) == ARG          # kind
    assert m(1, two, 2, FAKE, 1024, 1, 0, 0, None) == ARG          # narrow takes one source
    assert m(0, two, 0, FAKE, 1024, 1, 0, 0, None) == ARG
    assert m(0, ptrs(*[FAKE] * 17), 17, FAKE, 1024, 1, 0, 0, None) == ARG
    assert m(0, two, 2, FAKE, 1024, 9, 0, 0, None) == ARG          # workgroups per CU
    assert m(0, two, 2, FAKE, 1024, 1, 0, 2, None) == ARG          # prefetch is 0 or 1
    assert m(0, None, 2, FAKE, 1024, 1, 0, 0, None) == NULL
    assert m(0, two, 2, None, 1024, 1, 0, 0, None) == NULL
    assert m(0, ptrs(FAKE, 0), 2, FAKE, 1024, 1, 0, 0, None) == NULL
    assert m(0, ptrs(FAKE, FAKE + 8), 2, FAKE, 1024, 1, 0, 0, None) == ALIGN
    assert m(2, ptrs(FAKE), 1, FAKE, 1000, 1, 0, 0, None) == ALIGN  # bytes % 16
    assert m(0, two, 2, FAKE, 0, 1, 0, 0, None) == OK               # nothing to do
    c = L.rxtest_copy_streams
    d2 = ptrs(FAKE + 8192, FAKE + 12288)
    assert c(two, d2, 0, 0, 1024, 1, 64, None) == ARG            # stream count
    assert c(ptrs(*[FAKE] * 17), ptrs(*[FAKE] * 17), 17, 0, 1024, 1, 64, None) == ARG
    assert c(two, d2, 2, 0, 1024, 3, 64, None) == ARG            # lanes
    assert c(two, d2, 2, 0, 1024, 1, 96, None) == ARG            # workgroup size
    assert c(None, d2, 2, 0, 1024, 1, 64, None) == NULL
    assert c(two, None, 2, 0, 1024, 1, 64, None) == NULL
    assert c(two, ptrs(FAKE, 0), 2, 0, 1024, 1, 64, None) == NULL
    assert c(two, ptrs(FAKE, FAKE + 8), 2, 0, 1024, 1, 64, None) == ALIGN
    assert c(two, d2, 2, 8, 1024, 1, 64, None) == ALIGN          # offset % 16
    assert c(two, d2, 2, 0, 1000, 2, 128, None) == ALIGN         # bytes % 16
    assert c(two, d2, 2, 16, 0, 2, 256, None) == OK              # nothing to do


def test_binding_fails_loudly_without_the_library(tmp_path):
    """No CPU fallback: with librx.so absent every entry point raises."""
    import subprocess
    import sys
    code = ("import allreduce_reduction_rx_amd as rx\n"
            "rx.lib_path = lambda: '/nonexistent/librx.so'\n"
            "rx._lib = None\n"
            "try:\n"
            "    rx.rx_status_string(0)\n"
            "except RuntimeError as e:\n"
            "    assert 'missing' in str(e)\n"
            "    print('raised')\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "raised"
