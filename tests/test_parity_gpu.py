"""GPU parity: every librx entry point against the CPU oracle, bit for bit
(FP32 sums at fixed source order reach the oracle exactly, BF16 narrowing
and FP8 codes and scales are exact), through the C ABI.

Workloads (named in rxgen): the RCCLX article's rank-id example
(code-journey.com, "Practical guide"), a decode-size flat reduce, the DDA
tree step on 4 MiB messages, and the two >= 16 MB low-precision messages
("Core feature 2: Low-Precision Collectives").
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import allreduce_reduction_rx_amd as rx
import oracle as O
import rxgen as G
from gpu_util import (DEV, Guarded, bits_equal, empty_like_np, first_mismatch, log,
                      to_gpu, to_host)

pytestmark = pytest.mark.gpu

NP = {O.FP32: np.float32, O.BF16: np.uint16}
TD = {O.FP32: torch.float32, O.BF16: torch.bfloat16}
FMTS = {O.E4M3: "e4m3", O.E5M2: "e5m2"}

SHAPES = [1, 2, 3, 7, 8, 9, 15, 16, 17, 127, 128, 129, 255, 256, 257, 1000, 4133, 70001]


def sync():
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# DDA flat
# ---------------------------------------------------------------------------

def test_flat_rank_id_example():
    w = G.WORKLOADS["flat_rank"]
    log("flat_rank")
    srcs = w.sources()
    dst = torch.empty(w.count, dtype=torch.float32, device=DEV)
    rx.rx_reduce_flat([to_gpu(s) for s in srcs], dst)
    sync()
    assert torch.all(dst == 28.0).item()


@pytest.mark.parametrize("name", ["flat_uniform", "decode"])
def test_flat_workloads(name):
    w = G.WORKLOADS[name]
    log(f"flat workload {name}")
    srcs = w.sources()
    g = Guarded(w.count, TD[w.dtype])
    rx.rx_reduce_flat([to_gpu(s) for s in srcs], g.t)
    sync()
    ref = O.reduce_flat(srcs, w.dtype)
    got = to_host(g.t)
    assert bits_equal(got, ref), first_mismatch(got, ref)
    assert g.guards_intact()


@pytest.mark.parametrize("dtype", [O.FP32, O.BF16])
@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 13, 16])
def test_flat_shapes(n, dtype):
    for count in SHAPES:
        log(f"flat n={n} dtype={dtype} count={count}")
        srcs = [G.fill(count, dtype, G.NORMAL_OUTLIER, seed=1000 + count, rank=r) for r in range(n)]
        g = Guarded(count, TD[dtype])
        rx.rx_reduce_flat([to_gpu(s) for s in srcs], g.t)
        sync()
        ref = O.reduce_flat(srcs, dtype)
        got = to_host(g.t)
        assert bits_equal(got, ref), f"count={count}: " + first_mismatch(got, ref)
        assert g.guards_intact(), f"count={count}: guard overwritten"


@pytest.mark.parametrize("dtype", [O.FP32, O.BF16])
def test_flat_in_place(dtype):
    n, count = 8, 100_003
    srcs = [G.fill(count, dtype, G.NORMAL, seed=77, rank=r) for r in range(n)]
    ref = O.reduce_flat(srcs, dtype)
    for j in (0, 5, 7):
        ts = [to_gpu(s) for s in srcs]
        rx.rx_reduce_flat(ts, ts[j])
        sync()
        got = to_host(ts[j])
        assert bits_equal(got, ref), f"alias {j}: " + first_mismatch(got, ref)


@pytest.mark.parametrize("dtype", [O.FP32, O.BF16])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 8, 13, 16])
@pytest.mark.parametrize("extra", [5, 1021 * 8 + 3])
@pytest.mark.parametrize("mib", [3, 9])
def test_flat_large_variant_ragged(n, dtype, extra, mib):
    # above the decode-size threshold. 3M elements: medium (up to 16 whole
    # tiles per CU on a 256-CU MI355X), a wave per whole tile for up to 8
    # sources; 9M: large, wave tiles with deferred stores and a grid-stride
    # loop (whole tiles only for few sources or FP32 up to 8); 13 and 16
    # sources the checked tile kernel at both sizes; the rest of the message
    # in a second launch; ragged element tail; also in place
    count = mib * (1 << 20) + extra
    srcs = [G.fill(count, dtype, G.NORMAL_OUTLIER, seed=1500 + n, rank=r) for r in range(n)]
    ref = O.reduce_flat(srcs, dtype)
    g = Guarded(count, TD[dtype])
    ts = [to_gpu(s) for s in srcs]
    log(f"flat large n={n} dtype={dtype} count={count}")
    rx.rx_reduce_flat(ts, g.t)
    sync()
    got = to_host(g.t)
    assert bits_equal(got, ref), first_mismatch(got, ref)
    assert g.guards_intact()
    rx.rx_reduce_flat(ts, ts[n - 1])
    sync()
    got = to_host(ts[n - 1])
    assert bits_equal(got, ref), "in place: " + first_mismatch(got, ref)


def test_flat_order_and_accumulation():
    # FP32 left fold in source order: ((1e8 + 1) - 1e8) == 0 but
    # ((1e8 - 1e8) + 1) == 1; BF16 {256, 1 x 7} -> 264 needs FP32 accumulation.
    a = np.full(64, 1e8, np.float32)
    b = np.full(64, 1.0, np.float32)
    c = np.full(64, -1e8, np.float32)
    for order, want in (((a, b, c), 0.0), ((a, c, b), 1.0)):
        dst = torch.empty(64, dtype=torch.float32, device=DEV)
        rx.rx_reduce_flat([to_gpu(x) for x in order], dst)
        sync()
        assert torch.all(dst == want).item()
    vals = [torch.full((40,), v, dtype=torch.bfloat16, device=DEV) for v in [256.0] + [1.0] * 7]
    dst = torch.empty(40, dtype=torch.bfloat16, device=DEV)
    rx.rx_reduce_flat(vals, dst)
    sync()
    assert torch.all(dst.float() == 264.0).item()


def test_flat_deterministic():
    w = G.WORKLOADS["decode"]
    ts = [to_gpu(s) for s in w.sources()]
    outs = []
    for _ in range(3):
        d = torch.empty(w.count, dtype=torch.bfloat16, device=DEV)
        rx.rx_reduce_flat(ts, d)
        outs.append(d)
    sync()
    assert all(torch.equal(outs[0].view(torch.int16), o.view(torch.int16)) for o in outs)


# ---------------------------------------------------------------------------
# DDA tree
# ---------------------------------------------------------------------------

def _tree_case(srcs, dtype, count, rank):
    n = len(srcs)
    gs = [Guarded(count, TD[dtype]) for _ in range(n)]   # interior holds a sentinel too
    sentinel = [to_host(g.t).copy() for g in gs]
    rx.rx_reduce_scatter_chunk_bcast([to_gpu(s) for s in srcs], rank, [g.t for g in gs])
    sync()
    ref = [s.copy() for s in sentinel]
    O.reduce_scatter_chunk_bcast(srcs, dtype, rank, ref)
    for j, g in enumerate(gs):
        got = to_host(g.t)
        assert bits_equal(got, ref[j]), f"rank={rank} dst={j}: " + first_mismatch(got, ref[j])
        assert g.guards_intact()


def test_tree_workload_all_ranks():
    w = G.WORKLOADS["tree"]
    srcs = w.sources()
    for k in range(w.nsrc):
        log(f"tree workload rank={k}")
        _tree_case(srcs, w.dtype, w.count, k)


@pytest.mark.parametrize("dtype", [O.FP32, O.BF16])
@pytest.mark.parametrize("n", [1, 3, 8, 16])
def test_tree_shapes(n, dtype):
    for count in [1, 7, 8, 9, 33, 127, 1000, 4133]:
        srcs = [G.fill(count, dtype, G.NORMAL, seed=2000 + count, rank=r) for r in range(n)]
        for k in range(n):
            log(f"tree n={n} dtype={dtype} count={count} rank={k}")
            _tree_case(srcs, dtype, count, k)


@pytest.mark.parametrize("dtype", [O.FP32, O.BF16])
@pytest.mark.parametrize("n", [2, 5, 8, 16])
@pytest.mark.parametrize("tiles_per_cu", [6, 7, 8])
def test_tree_medium_band(n, dtype, tiles_per_cu):
    # chunks of 6 to 8 whole 64-vector tiles per CU on a 256-CU MI355X: a
    # wave per tile, then the rest of the chunk; ragged message end; ranks
    # 0 and 1 and the last (a short chunk, below the band)
    ve = 4 if dtype == O.FP32 else 8
    count = n * tiles_per_cu * 256 * 64 * ve + 9
    srcs = [G.fill(count, dtype, G.NORMAL, seed=2600 + 10 * n + tiles_per_cu, rank=r) for r in range(n)]
    for k in (0, 1, n - 1):
        log(f"tree medium n={n} dtype={dtype} tiles/CU={tiles_per_cu} rank={k}")
        _tree_case(srcs, dtype, count, k)
    # in place (the one-device TREE allreduce's use): sources are the
    # destinations
    k = 1
    log(f"tree medium in place n={n} dtype={dtype} tiles/CU={tiles_per_cu} rank={k}")
    ts = [to_gpu(s) for s in srcs]
    rx.rx_reduce_scatter_chunk_bcast(ts, k, ts)
    sync()
    ref = [s.copy() for s in srcs]
    O.reduce_scatter_chunk_bcast(srcs, dtype, k, ref)
    for j in range(n):
        got = to_host(ts[j])
        assert bits_equal(got, ref[j]), f"in place dst {j}: " + first_mismatch(got, ref[j])


@pytest.mark.parametrize("n", [3, 8])
def test_tree_large_fp32_whole_tiles(n):
    # FP32 chunks of 64 and more 64-vector tiles per CU on a 256-CU MI355X:
    # whole tiles with four 64-thread workgroups per CU, then the rest of the
    # chunk; ragged message end; ranks 0 and the last
    count = n * 64 * 256 * 64 * 4 + 9
    srcs = [G.fill(count, O.FP32, G.NORMAL, seed=2700 + n, rank=r) for r in range(n)]
    for k in (0, n - 1):
        log(f"tree large fp32 whole n={n} rank={k}")
        _tree_case(srcs, O.FP32, count, k)


@pytest.mark.parametrize("dtype", [O.FP32, O.BF16])
@pytest.mark.parametrize("n", [3, 8, 16])
def test_tree_large_variant_ragged(n, dtype):
    # chunks above the medium band (whole tiles and the rest of the chunk
    # for BF16; FP32 two lanes per vector), ragged message end; ranks 0 and 1
    # (chunks from the start and from inside the message) and the last (a
    # short chunk)
    count = n * (1 << 21) + 9
    srcs = [G.fill(count, dtype, G.NORMAL, seed=2500 + n, rank=r) for r in range(n)]
    for k in (0, 1, n - 1):
        log(f"tree large n={n} dtype={dtype} rank={k}")
        _tree_case(srcs, dtype, count, k)


@pytest.mark.parametrize("dtype", [O.FP32, O.BF16])
@pytest.mark.parametrize("extra_vectors,extra", [(0, 0), (0, 9), (1, 0), (1, 3)])
def test_tree_word_lane_boundary(dtype, extra_vectors, extra):
    # decode-size chunks: 4-byte-word lanes while the words fit six waves per
    # CU on a 256-CU MI355X (24,576 16-byte vectors), two lanes per vector
    # above; chunks at the limit and one vector past it, whole and ragged
    n = 8
    ve = 4 if dtype == O.FP32 else 8
    count = n * (24576 + extra_vectors) * ve + extra
    srcs = [G.fill(count, dtype, G.NORMAL, seed=2800 + 10 * extra_vectors + extra, rank=r) for r in range(n)]
    for k in (0, n - 1):
        log(f"tree word-lane boundary dtype={dtype} count={count} rank={k}")
        _tree_case(srcs, dtype, count, k)


def test_tree_in_place():
    n, count, dtype = 8, 65536 + 24, O.BF16
    srcs = [G.fill(count, dtype, G.NORMAL, seed=99, rank=r) for r in range(n)]
    for k in (0, 7):
        ts = [to_gpu(s) for s in srcs]
        rx.rx_reduce_scatter_chunk_bcast(ts, k, ts)
        sync()
        ref = [s.copy() for s in srcs]
        O.reduce_scatter_chunk_bcast(srcs, dtype, k, ref)
        for j in range(n):
            assert bits_equal(to_host(ts[j]), ref[j])


# ---------------------------------------------------------------------------
# Low-precision path
# ---------------------------------------------------------------------------

def _quant_gpu(srcs, dtype, fmt, block, count):
    nb = -(-count // block)
    codes = [Guarded(count, torch.uint8) for _ in srcs]
    scales = [Guarded(nb, torch.float32) for _ in srcs]
    rx.rx_quant_fp8([to_gpu(s) for s in srcs], FMTS[fmt], block,
                    [c.t for c in codes], [s.t for s in scales], count=count)
    sync()
    for g in codes + scales:
        assert g.guards_intact()
    return [to_host(c.t) for c in codes], [to_host(s.t) for s in scales]


@pytest.mark.parametrize("dtype", [O.FP32, O.BF16])
@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
@pytest.mark.parametrize("block", [32, 64, 128, 256, 512, 1024])
def test_quant_shapes(dtype, fmt, block):
    n = 3
    for count in [1, 5, 17, block - 1, block, block + 3, 4 * block + 7, 5000, 33_333]:
        log(f"quant dtype={dtype} fmt={fmt} block={block} count={count}")
        srcs = [G.fill(count, dtype, G.NORMAL_OUTLIER, seed=3000 + count, rank=r) for r in range(n)]
        gc, gs = _quant_gpu(srcs, dtype, fmt, block, count)
        rc, rs = O.quant_fp8(srcs, dtype, fmt, block)
        for j in range(n):
            assert bits_equal(gc[j], rc[j]), f"codes count={count} src={j}: " + first_mismatch(gc[j], rc[j])
            assert bits_equal(gs[j], rs[j]), f"scales count={count} src={j}: " + first_mismatch(gs[j], rs[j])


@pytest.mark.parametrize("dtype,fmt,block", [(O.FP32, O.E4M3, 128), (O.BF16, O.E5M2, 256),
                                             (O.FP32, O.E5M2, 1024), (O.BF16, O.E4M3, 32)])
def test_quant_decode_whole_tile_rows(dtype, fmt, block):
    # decode-size sources of whole tiles (the loop-free kernel, one grid row
    # per source, rows padded to a multiple of 8 workgroups of 4 tiles):
    # tile counts that leave the last workgroup partly idle or pad the row,
    # with 1 to 16 sources; unwritten codes or scales keep the sentinel
    ve = 4 if dtype == O.FP32 else 8
    lanes = block // ve
    tile = (1 if lanes <= 64 else lanes // 64) * 64 * ve
    for n in (1, 3, 8, 16):
        for t in (1, 2, 3, 4, 5, 7, 8, 9, 31, 32, 33, 37):
            count = t * tile
            log(f"quant whole-tile rows dtype={dtype} fmt={fmt} block={block} n={n} tiles={t}")
            srcs = [G.fill(count, dtype, G.NORMAL_OUTLIER, seed=3700 + 41 * t + n, rank=r) for r in range(n)]
            gc, gs = _quant_gpu(srcs, dtype, fmt, block, count)
            rc, rs = O.quant_fp8(srcs, dtype, fmt, block)
            for j in range(n):
                assert bits_equal(gc[j], rc[j]), f"codes n={n} tiles={t} src={j}: " + first_mismatch(gc[j], rc[j])
                assert bits_equal(gs[j], rs[j]), f"scales n={n} tiles={t} src={j}: " + first_mismatch(gs[j], rs[j])


@pytest.mark.parametrize("dtype,fmt,block,extra", [(O.BF16, O.E5M2, 256, 512), (O.BF16, O.E5M2, 256, 1536),
                                                   (O.FP32, O.E4M3, 128, 256), (O.FP32, O.E5M2, 64, 768)])
def test_quant_large_rest_whole_tiles(dtype, fmt, block, extra):
    # a large message (whole-tile kernel over 4-load tiles) whose rest is a
    # whole number of decode-size tiles: the rest runs the loop-free kernel
    # through pointers offset into the message
    n = 8
    count = 4 * 64 * (4 if dtype == O.FP32 else 8) * 256 + extra
    log(f"quant large rest whole tiles dtype={dtype} fmt={fmt} block={block} count={count}")
    srcs = [G.fill(count, dtype, G.NORMAL_OUTLIER, seed=3800 + extra, rank=r) for r in range(n)]
    gc, gs = _quant_gpu(srcs, dtype, fmt, block, count)
    rc, rs = O.quant_fp8(srcs, dtype, fmt, block)
    for j in range(n):
        assert bits_equal(gc[j], rc[j]), f"codes src={j}: " + first_mismatch(gc[j], rc[j])
        assert bits_equal(gs[j], rs[j]), f"scales src={j}: " + first_mismatch(gs[j], rs[j])


@pytest.mark.parametrize("dtype", [O.FP32, O.BF16])
@pytest.mark.parametrize("fmt,block", [(O.E4M3, 128), (O.E5M2, 256), (O.E4M3, 1024), (O.E5M2, 32)])
def test_quant_large_variant_ragged(dtype, fmt, block):
    # > 2048 large-variant tiles on a 256-CU MI355X: the 4-loads-per-lane
    # kernel with a grid-stride loop, ragged tail and partial last block
    count = 5 * (1 << 20) + 5
    log(f"quant large variant dtype={dtype} fmt={fmt} block={block}")
    srcs = [G.fill(count, dtype, G.NORMAL_OUTLIER, seed=3500 + block, rank=0)]
    gc, gs = _quant_gpu(srcs, dtype, fmt, block, count)
    rc, rs = O.quant_fp8(srcs, dtype, fmt, block)
    assert bits_equal(gc[0], rc[0]), first_mismatch(gc[0], rc[0])
    assert bits_equal(gs[0], rs[0]), first_mismatch(gs[0], rs[0])


@pytest.mark.parametrize("dtype,fmt,block,mib", [(O.FP32, O.E4M3, 128, 32), (O.BF16, O.E5M2, 1024, 32),
                                                 (O.FP32, O.E4M3, 128, 128), (O.BF16, O.E5M2, 1024, 128),
                                                 (O.FP32, O.E5M2, 1024, 128), (O.BF16, O.E4M3, 32, 128)])
def test_quant_whole_tiles_ragged(dtype, fmt, block, mib):
    # 8 sources of mib MiB + 5 elements on a 256-CU MI355X: the whole-tile
    # kernel with 4 loads per lane (32 MiB) or 8 loads per lane and the next
    # tile prefetched (128 MiB: 1 GiB of input), blocks of one and of several
    # loads, then the ragged end of every source (a partial last block) in a
    # second launch. Every code and scale against the oracle, which runs over
    # windows of whole blocks in a thread pool.
    n = 8
    count = mib * (1 << 20) // (4 if dtype == O.FP32 else 2) + 5
    log(f"quant whole tiles dtype={dtype} fmt={fmt} block={block} count={count}")
    srcs = [G.fill(count, dtype, G.NORMAL_OUTLIER, seed=3600 + block + mib, rank=r) for r in range(n)]
    gc, gs = _quant_gpu(srcs, dtype, fmt, block, count)
    win = 8192 * block

    def check(i0):
        i1 = min(i0 + win, count)
        b0, b1 = i0 // block, -(-i1 // block)
        rc, rs = O.quant_fp8([x[i0:i1] for x in srcs], dtype, fmt, block)
        for j in range(n):
            if not bits_equal(gc[j][i0:i1], rc[j]):
                return f"codes src={j} window [{i0}, {i1}): " + first_mismatch(gc[j][i0:i1], rc[j])
            if not bits_equal(gs[j][b0:b1], rs[j]):
                return f"scales src={j} window [{i0}, {i1}): " + first_mismatch(gs[j][b0:b1], rs[j])
        return None

    with ThreadPoolExecutor(_pool_size()) as ex:
        for res in ex.map(check, range(0, count, win)):
            assert res is None, res


@pytest.mark.parametrize("dtype,fmt,block", [(O.FP32, O.E4M3, 64), (O.BF16, O.E5M2, 512)])
def test_quant_sixteen_sources_large(dtype, fmt, block):
    # 16 sources (the most the argument tables hold) above the decode-size
    # threshold: tile t of the whole-tile kernel belongs to source
    # t / tiles_per_source, the ragged end of every source in a second launch
    n = 16
    count = (1 << 20) + 3 * block + 11
    log(f"quant 16 sources dtype={dtype} fmt={fmt} block={block} count={count}")
    srcs = [G.fill(count, dtype, G.NORMAL_OUTLIER, seed=3700 + r, rank=r) for r in range(n)]
    gc, gs = _quant_gpu(srcs, dtype, fmt, block, count)
    rc, rs = O.quant_fp8(srcs, dtype, fmt, block)
    for j in range(n):
        assert bits_equal(gc[j], rc[j]), f"codes src={j}: " + first_mismatch(gc[j], rc[j])
        assert bits_equal(gs[j], rs[j]), f"scales src={j}: " + first_mismatch(gs[j], rs[j])


def test_quant_degenerate_blocks():
    # zero blocks, tiny blocks (FMAX / A overflows), huge values, -0
    count, block = 1024, 128
    x = np.zeros(count, np.float32)
    x[128:256] = np.float32(1e-40) * (np.arange(128) % 3 - 1)
    x[256:384] = np.float32(3e38) * np.where(np.arange(128) % 2 == 0, 1, -1)
    x[384:512] = -0.0
    x[512:640] = np.float32(2.0 ** -140)
    x[640:768] = 448.0
    x[768:] = np.linspace(-1, 1, 256, dtype=np.float32)
    for fmt in (O.E4M3, O.E5M2):
        gc, gs = _quant_gpu([x], O.FP32, fmt, block, count)
        rc, rs = O.quant_fp8([x], O.FP32, fmt, block)
        assert bits_equal(gc[0], rc[0]), first_mismatch(gc[0], rc[0])
        assert bits_equal(gs[0], rs[0]), first_mismatch(gs[0], rs[0])


def _drr_gpu(codes, scales, fmt, block, mode, hp_dtype, want_hp, count):
    nb = -(-count // block)
    oc = os_ = hp = None
    if mode == O.DRR_REQUANT:
        oc = Guarded(count, torch.uint8)
        os_ = Guarded(nb, torch.float32)
    if mode == O.DRR_SUM or want_hp:
        hp = Guarded(count, TD[hp_dtype])
    rx.rx_dequant_reduce_requant([to_gpu(c) for c in codes], [to_gpu(s) for s in scales],
                                 FMTS[fmt], block, mode,
                                 None if oc is None else oc.t, None if os_ is None else os_.t,
                                 None if hp is None else hp.t, count=count)
    sync()
    out = []
    for g in (oc, os_, hp):
        if g is None:
            out.append(None)
        else:
            assert g.guards_intact()
            out.append(to_host(g.t))
    return out


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
@pytest.mark.parametrize("block", [32, 128, 256, 1024])
@pytest.mark.parametrize("n", [1, 2, 8, 16])
def test_drr_shapes(fmt, block, n):
    for count in [1, 15, 16, 17, block + 5, 3 * block, 5000, 40_001]:
        srcs = [G.fill(count, O.FP32, G.LAPLACE, seed=4000 + count, rank=r) for r in range(n)]
        codes, scales = O.quant_fp8(srcs, O.FP32, fmt, block)
        for mode, hp_dtype, want_hp in ((O.DRR_SUM, O.FP32, True), (O.DRR_SUM, O.BF16, True),
                                        (O.DRR_REQUANT, O.FP32, False),
                                        (O.DRR_REQUANT, O.FP32, True),
                                        (O.DRR_REQUANT, O.BF16, True)):
            log(f"drr fmt={fmt} block={block} n={n} count={count} mode={mode} hp={hp_dtype}/{want_hp}")
            got = _drr_gpu(codes, scales, fmt, block, mode, hp_dtype, want_hp, count)
            ref = O.dequant_reduce_requant(codes, scales, fmt, block, mode, hp_dtype, want_hp)
            for name, g, r in zip(("codes", "scales", "hp"), got, ref):
                assert (g is None) == (r is None)
                if g is not None:
                    assert bits_equal(g, r), f"{name} count={count}: " + first_mismatch(g, r)


@pytest.mark.parametrize("fmt,block", [(O.E4M3, 128), (O.E5M2, 256), (O.E4M3, 1024)])
def test_drr_codes_only_two_per_cu(fmt, block):
    # code-only output with at least 32 tiles of 1024 codes per CU on a
    # 256-CU MI355X: 16 x 1 layout, two workgroups per CU, each XCD a
    # contiguous range of tiles; ragged tail and partial last block
    n, count = 3, 8 * (1 << 20) + 7
    srcs = [G.fill(count, O.FP32, G.LAPLACE, seed=4600 + block, rank=r) for r in range(n)]
    codes, scales = O.quant_fp8(srcs, O.FP32, fmt, block)
    log(f"drr codes only fmt={fmt} block={block} count={count}")
    got = _drr_gpu(codes, scales, fmt, block, O.DRR_REQUANT, O.FP32, False, count)
    ref = O.dequant_reduce_requant(codes, scales, fmt, block, O.DRR_REQUANT, O.FP32, False)
    for name, g, r in zip(("codes", "scales", "hp"), got, ref):
        assert (g is None) == (r is None)
        if g is not None:
            assert bits_equal(g, r), f"{name}: " + first_mismatch(g, r)


@pytest.mark.parametrize("n", [2, 5, 13, 16])
def test_drr_staged_output_source_counts(n):
    # FP32 and BF16 outputs from several sources at large sizes run the 16 x 1
    # layout with the output staged through LDS: each source count is a
    # kernel instance of its own; whole tiles through the stage, the ragged
    # last tile directly
    count = (1 << 20) + 13
    for fmt, block in ((O.E4M3, 128), (O.E5M2, 1024)):
        srcs = [G.fill(count, O.FP32, G.LAPLACE, seed=4700 + n + block, rank=r) for r in range(n)]
        codes, scales = O.quant_fp8(srcs, O.FP32, fmt, block)
        for mode, hp_dtype in ((O.DRR_SUM, O.FP32), (O.DRR_SUM, O.BF16), (O.DRR_REQUANT, O.FP32),
                               (O.DRR_REQUANT, O.BF16)):
            log(f"drr staged output n={n} fmt={fmt} block={block} mode={mode} hp={hp_dtype}")
            got = _drr_gpu(codes, scales, fmt, block, mode, hp_dtype, True, count)
            ref = O.dequant_reduce_requant(codes, scales, fmt, block, mode, hp_dtype, True)
            for name, g, r in zip(("codes", "scales", "hp"), got, ref):
                assert (g is None) == (r is None)
                if g is not None:
                    assert bits_equal(g, r), f"{name}: " + first_mismatch(g, r)


@pytest.mark.parametrize("fmt,block", [(O.E4M3, 128), (O.E5M2, 256), (O.E4M3, 32),
                                       (O.E5M2, 512), (O.E4M3, 1024)])
def test_drr_large_variant_ragged(fmt, block):
    # > 1024 tiles of 1024 codes: the grid-stride kernels in every chunk
    # layout (16 codes x 1 for code-only output, 8 x 2 for BF16 output, 4 x 4
    # for FP32 output), ragged tail and partial last block
    n, count = 4, (1 << 21) + 7
    srcs = [G.fill(count, O.FP32, G.LAPLACE, seed=4500 + block, rank=r) for r in range(n)]
    codes, scales = O.quant_fp8(srcs, O.FP32, fmt, block)
    for mode, hp_dtype, want_hp in ((O.DRR_SUM, O.BF16, True), (O.DRR_SUM, O.FP32, True),
                                    (O.DRR_REQUANT, O.FP32, False), (O.DRR_REQUANT, O.BF16, True),
                                    (O.DRR_REQUANT, O.FP32, True)):
        log(f"drr large variant fmt={fmt} block={block} mode={mode} hp={hp_dtype}/{want_hp}")
        got = _drr_gpu(codes, scales, fmt, block, mode, hp_dtype, want_hp, count)
        ref = O.dequant_reduce_requant(codes, scales, fmt, block, mode, hp_dtype, want_hp)
        for name, g, r in zip(("codes", "scales", "hp"), got, ref):
            assert (g is None) == (r is None)
            if g is not None:
                assert bits_equal(g, r), f"{name}: " + first_mismatch(g, r)


@pytest.mark.parametrize("fmt,block", [(O.E4M3, 128), (O.E5M2, 256), (O.E4M3, 32),
                                       (O.E5M2, 512), (O.E4M3, 1024)])
def test_drr_one_source_large_ragged(fmt, block):
    # one source above the decode-size threshold (the separate
    # dequantization and a one-source requantization): whole tiles in the
    # 4 x 4 (FP32 output, blocks up to 256), 8 x 2 (BF16 output, blocks up
    # to 512) or 16 x 1 layout, then the ragged remainder in a second launch
    count = (1 << 21) + 1000 * 8 + 7
    srcs = [G.fill(count, O.FP32, G.LAPLACE, seed=4800 + block, rank=0)]
    codes, scales = O.quant_fp8(srcs, O.FP32, fmt, block)
    for mode, hp_dtype, want_hp in ((O.DRR_SUM, O.BF16, True), (O.DRR_SUM, O.FP32, True),
                                    (O.DRR_REQUANT, O.FP32, False), (O.DRR_REQUANT, O.BF16, True),
                                    (O.DRR_REQUANT, O.FP32, True)):
        log(f"drr one source fmt={fmt} block={block} mode={mode} hp={hp_dtype}/{want_hp}")
        got = _drr_gpu(codes, scales, fmt, block, mode, hp_dtype, want_hp, count)
        ref = O.dequant_reduce_requant(codes, scales, fmt, block, mode, hp_dtype, want_hp)
        for name, g, r in zip(("codes", "scales", "hp"), got, ref):
            assert (g is None) == (r is None)
            if g is not None:
                assert bits_equal(g, r), f"{name}: " + first_mismatch(g, r)


def test_drr_codes_only_prefetch_ragged():
    """Codes only from 8 sources at 512 tiles of 1024 codes per CU and more
    (on a 256-CU MI355X): the prefetching whole-tile kernel at one workgroup
    per CU, then the ragged remainder. The codes come from the GPU's
    quantizer on rxgen input and are checked against the oracle's quantizer
    first; DRR is then compared with the oracle's DRR of the oracle's codes,
    every code and scale, in windows of whole blocks on a thread pool."""
    n, fmt, block = 8, O.E4M3, 128
    count = (1 << 27) + 5003
    nb = -(-count // block)
    log(f"drr codes only prefetch count={count}")
    srcs = [G.fill(count, O.BF16, G.LAPLACE, seed=4900 + r, rank=r) for r in range(n)]
    ts = [to_gpu(x) for x in srcs]
    codes = [torch.empty(count, dtype=torch.uint8, device=DEV) for _ in range(n)]
    scales = [torch.empty(nb, dtype=torch.float32, device=DEV) for _ in range(n)]
    rx.rx_quant_fp8(ts, FMTS[fmt], block, codes, scales)
    del ts
    oc = Guarded(count, torch.uint8)
    osc = Guarded(nb, torch.float32)
    rx.rx_dequant_reduce_requant(codes, scales, FMTS[fmt], block, rx.RX_DRR_REQUANT, oc.t, osc.t)
    sync()
    assert oc.guards_intact() and osc.guards_intact()
    g_codes = [c.cpu().numpy() for c in codes]
    g_scales = [q.cpu().numpy() for q in scales]
    g_oc, g_os = to_host(oc.t), to_host(osc.t)
    del codes, scales, oc, osc
    torch.cuda.empty_cache()
    win = 8192 * block

    def check(i0):
        i1 = min(i0 + win, count)
        b0, b1 = i0 // block, -(-i1 // block)
        rc, rs = O.quant_fp8([x[i0:i1] for x in srcs], O.BF16, fmt, block)
        for r in range(n):
            if not bits_equal(g_codes[r][i0:i1], rc[r]) or not bits_equal(g_scales[r][b0:b1], rs[r]):
                return f"quantizer rank {r} window [{i0}, {i1})"
        r_oc, r_os, _ = O.dequant_reduce_requant(rc, rs, fmt, block, O.DRR_REQUANT, O.FP32, False)
        if not bits_equal(g_oc[i0:i1], r_oc):
            return f"codes window [{i0}, {i1}): " + first_mismatch(g_oc[i0:i1], r_oc)
        if not bits_equal(g_os[b0:b1], r_os):
            return f"scales window [{i0}, {i1}): " + first_mismatch(g_os[b0:b1], r_os)
        return None

    with ThreadPoolExecutor(_pool_size()) as ex:
        for res in ex.map(check, range(0, count, win)):
            assert res is None, res


@pytest.mark.parametrize("hp_dtype", [O.FP32, O.BF16])
def test_drr_staged_prefetch_ragged(hp_dtype):
    """Requantization with the high-precision output staged, at 256 tiles of
    1024 codes per CU and more (on a 256-CU MI355X): the prefetching staged
    kernel at one workgroup per CU, then the ragged remainder. GPU quantizer
    output checked against the oracle's first; DRR's codes, scales and output
    against the oracle's DRR of the oracle's codes, in windows of whole
    blocks on a thread pool."""
    n, fmt, block = 3, O.E4M3, 128
    count = (1 << 26) + 5003
    nb = -(-count // block)
    log(f"drr staged prefetch hp={hp_dtype} count={count}")
    srcs = [G.fill(count, O.FP32, G.LAPLACE, seed=4950 + r, rank=r) for r in range(n)]
    ts = [to_gpu(x) for x in srcs]
    codes = [torch.empty(count, dtype=torch.uint8, device=DEV) for _ in range(n)]
    scales = [torch.empty(nb, dtype=torch.float32, device=DEV) for _ in range(n)]
    rx.rx_quant_fp8(ts, FMTS[fmt], block, codes, scales)
    del ts
    oc = Guarded(count, torch.uint8)
    osc = Guarded(nb, torch.float32)
    hp = Guarded(count, TD[hp_dtype])
    rx.rx_dequant_reduce_requant(codes, scales, FMTS[fmt], block, rx.RX_DRR_REQUANT, oc.t, osc.t, hp.t)
    sync()
    assert oc.guards_intact() and osc.guards_intact() and hp.guards_intact()
    g_codes = [c.cpu().numpy() for c in codes]
    g_scales = [q.cpu().numpy() for q in scales]
    g_oc, g_os, g_hp = to_host(oc.t), to_host(osc.t), to_host(hp.t)
    del codes, scales, oc, osc, hp
    torch.cuda.empty_cache()
    win = 8192 * block

    def check(i0):
        i1 = min(i0 + win, count)
        b0, b1 = i0 // block, -(-i1 // block)
        rc, rs = O.quant_fp8([x[i0:i1] for x in srcs], O.FP32, fmt, block)
        for r in range(n):
            if not bits_equal(g_codes[r][i0:i1], rc[r]) or not bits_equal(g_scales[r][b0:b1], rs[r]):
                return f"quantizer rank {r} window [{i0}, {i1})"
        r_oc, r_os, r_hp = O.dequant_reduce_requant(rc, rs, fmt, block, O.DRR_REQUANT, hp_dtype, True)
        for name, g_, r_ in (("codes", g_oc[i0:i1], r_oc), ("scales", g_os[b0:b1], r_os), ("hp", g_hp[i0:i1], r_hp)):
            if not bits_equal(g_, r_):
                return f"{name} window [{i0}, {i1}): " + first_mismatch(g_, r_)
        return None

    with ThreadPoolExecutor(_pool_size()) as ex:
        for res in ex.map(check, range(0, count, win)):
            assert res is None, res


@pytest.mark.parametrize("fmt,block", [(O.E4M3, 128), (O.E5M2, 256), (O.E4M3, 32)])
@pytest.mark.parametrize("n", [1, 3, 8, 16])
def test_drr_decode_whole_tiles(fmt, block, n):
    # decode-size ranges of whole 256-code tiles (the loop-free kernel): every
    # mode and output type, and the LP tree step's chunks, which start inside
    # the message
    count = 256 * 96
    srcs = [G.fill(count, O.FP32, G.LAPLACE, seed=4990 + n + block, rank=r) for r in range(n)]
    codes, scales = O.quant_fp8(srcs, O.FP32, fmt, block)
    for mode, hp_dtype, want_hp in ((O.DRR_SUM, O.BF16, True), (O.DRR_SUM, O.FP32, True),
                                    (O.DRR_REQUANT, O.FP32, False), (O.DRR_REQUANT, O.BF16, True),
                                    (O.DRR_REQUANT, O.FP32, True)):
        log(f"drr decode whole tiles fmt={fmt} block={block} n={n} mode={mode} hp={hp_dtype}/{want_hp}")
        got = _drr_gpu(codes, scales, fmt, block, mode, hp_dtype, want_hp, count)
        ref = O.dequant_reduce_requant(codes, scales, fmt, block, mode, hp_dtype, want_hp)
        for name, g, r in zip(("codes", "scales", "hp"), got, ref):
            assert (g is None) == (r is None)
            if g is not None:
                assert bits_equal(g, r), f"mode={mode} {name}: " + first_mismatch(g, r)
    for k in range(n):
        log(f"lp tree decode whole tiles fmt={fmt} block={block} n={n} rank={k}")
        _lp_tree_case(codes, scales, fmt, block, k, count, hp_dtype=(None, O.BF16, O.FP32)[k % 3])


@pytest.mark.parametrize("fmt,block", [(O.E4M3, 128), (O.E5M2, 512)])
def test_lp_tree_large_variant_ragged(fmt, block):
    # chunks above the decode-size threshold, ragged message end
    n, count = 3, 3 * (1 << 21) + 5
    srcs = [G.fill(count, O.FP32, G.NORMAL_OUTLIER, seed=5500 + block, rank=r) for r in range(n)]
    codes, scales = O.quant_fp8(srcs, O.FP32, fmt, block)
    for k in range(n):
        log(f"lp tree large variant fmt={fmt} block={block} rank={k}")
        _lp_tree_case(codes, scales, fmt, block, k, count,
                      hp_dtype=(O.BF16, None, O.FP32)[k % 3])


def _lp_tree_case(codes, scales, fmt, block, rank, count, hp_dtype=None):
    n = len(codes)
    nb = -(-count // block)
    dc = [Guarded(count, torch.uint8) for _ in range(n)]
    ds = [Guarded(nb, torch.float32) for _ in range(n)]
    hp = None if hp_dtype is None else Guarded(count, TD[hp_dtype])
    ref_c = [to_host(g.t).copy() for g in dc]
    ref_s = [to_host(g.t).copy() for g in ds]
    ref_h = None if hp is None else to_host(hp.t).copy()
    rx.rx_lp_reduce_scatter_chunk_bcast([to_gpu(c) for c in codes], [to_gpu(s) for s in scales],
                                        FMTS[fmt], block, rank, [g.t for g in dc], [g.t for g in ds],
                                        None if hp is None else hp.t, count=count)
    sync()
    O.lp_reduce_scatter_chunk_bcast(codes, scales, fmt, block, rank, ref_c, ref_s,
                                    ref_h, O.FP32 if hp_dtype is None else hp_dtype)
    for j in range(n):
        got_c, got_s = to_host(dc[j].t), to_host(ds[j].t)
        assert bits_equal(got_c, ref_c[j]), f"rank={rank} dst={j} codes: " + first_mismatch(got_c, ref_c[j])
        assert bits_equal(got_s, ref_s[j]), f"rank={rank} dst={j} scales: " + first_mismatch(got_s, ref_s[j])
        assert dc[j].guards_intact() and ds[j].guards_intact()
    if hp is not None:
        got_h = to_host(hp.t)
        assert bits_equal(got_h, ref_h), f"rank={rank} hp: " + first_mismatch(got_h, ref_h)
        assert hp.guards_intact()


@pytest.mark.parametrize("fmt,block", [(O.E4M3, 128), (O.E5M2, 256), (O.E4M3, 32), (O.E5M2, 1024)])
@pytest.mark.parametrize("n", [1, 3, 8, 16])
def test_lp_tree_shapes(fmt, block, n):
    for count in [1, 17, block, 3 * block + 5, 20_000, 300_001]:
        srcs = [G.fill(count, O.FP32, G.NORMAL_OUTLIER, seed=5000 + count, rank=r) for r in range(n)]
        codes, scales = O.quant_fp8(srcs, O.FP32, fmt, block)
        for k in range(n):
            log(f"lp tree fmt={fmt} block={block} n={n} count={count} rank={k}")
            _lp_tree_case(codes, scales, fmt, block, k, count,
                          hp_dtype=(O.BF16, None, O.FP32)[k % 3])


def test_lp_tree_fp32_workload_all_ranks():
    """The low-precision tree step on the 8 x 64 MiB FP32 message (E4M3,
    blocks of 128): each rank's 2,097,152-element chunk (the large variant)."""
    w = G.WORKLOADS["lp_fp32"]
    fmt, block = O.FMT[w.fp8], w.block
    srcs = w.sources()
    codes, scales = O.quant_fp8(srcs, w.dtype, fmt, block)
    del srcs
    for k in range(w.nsrc):
        log(f"lp tree lp_fp32 rank={k}")
        _lp_tree_case(codes, scales, fmt, block, k, w.count, hp_dtype=O.FP32 if k == 0 else None)


def test_lp_fp32_workload_full():
    """Low-precision allreduce on 8 x 16,777,216 FP32 (N(0,1), 1% outliers
    x100), E4M3, blocks of 128: the flat reduce, the tree step of rank 3,
    quant and DRR-REQUANT (+FP32 output) compared in full."""
    w = G.WORKLOADS["lp_fp32"]
    fmt, block = O.FMT[w.fp8], w.block
    log("lp_fp32 generate")
    srcs = w.sources()
    log("lp_fp32 gpu")
    gc, gs = _quant_gpu(srcs, w.dtype, fmt, block, w.count)
    log("lp_fp32 oracle quant")
    rc, rs = O.quant_fp8(srcs, w.dtype, fmt, block)
    for j in range(w.nsrc):
        assert bits_equal(gc[j], rc[j]), f"codes src={j}: " + first_mismatch(gc[j], rc[j])
        assert bits_equal(gs[j], rs[j]), f"scales src={j}: " + first_mismatch(gs[j], rs[j])
    del gc, gs
    log("lp_fp32 drr")
    oc, osc, hp = _drr_gpu(rc, rs, fmt, block, O.DRR_REQUANT, O.FP32, True, w.count)
    r_oc, r_os, r_hp = O.dequant_reduce_requant(rc, rs, fmt, block, O.DRR_REQUANT, O.FP32, True)
    assert bits_equal(oc, r_oc), first_mismatch(oc, r_oc)
    assert bits_equal(osc, r_os), first_mismatch(osc, r_os)
    assert bits_equal(hp, r_hp), first_mismatch(hp, r_hp)
    # the full-precision legs of the same message: flat reduce in full, and
    # the tree step of rank 3 (its chunk in all 8 destinations, nothing else)
    log("lp_fp32 flat + tree")
    T32 = O.reduce_flat(srcs, O.FP32)
    ts = [to_gpu(x) for x in srcs]
    flat = torch.empty(w.count, dtype=torch.float32, device=DEV)
    rx.rx_reduce_flat(ts, flat)
    sync()
    got = to_host(flat)
    assert bits_equal(got, T32), first_mismatch(got, T32)
    del flat, got
    k = 3
    lo, hi = O.tree_chunk(w.count, w.nsrc, O.FP32, k)
    dsts = [torch.zeros(w.count, dtype=torch.float32, device=DEV) for _ in range(w.nsrc)]
    rx.rx_reduce_scatter_chunk_bcast(ts, k, dsts)
    sync()
    want = torch.from_numpy(T32[lo:hi]).to(DEV)
    for j, d in enumerate(dsts):
        assert torch.equal(d[lo:hi].view(torch.int32), want.view(torch.int32)), f"tree dst {j}"
        assert not d[:lo].view(torch.int32).any().item() and not d[hi:].view(torch.int32).any().item()
    del ts, dsts, want
    torch.cuda.empty_cache()
    # end-to-end error against the unquantized FP32 sum: N * 2^-4 * blockabsmax
    T = T32.astype(np.float64)
    X_absmax = np.zeros(w.count // block)
    for s in srcs:
        X_absmax = np.maximum(X_absmax, np.abs(s.astype(np.float64)).reshape(-1, block).max(axis=1))
    bound = w.nsrc * 2.0 ** -4 * np.repeat(X_absmax, block)
    err = np.abs(hp.astype(np.float64) - T)
    log(f"lp_fp32 max err/bound = {np.max(err / bound):.4f}")
    assert np.all(err <= bound)


def _pool_size() -> int:
    # the GPU machine's CPU share is 16 threads, whatever os.cpu_count() shows
    return max(1, min(16, os.cpu_count() or 1))


def test_lp_bf16_workload_full():
    """Low-precision large message: 8 x 268,435,456 BF16 (Laplace(0,1)),
    E5M2, blocks of 256, in the launch configuration the benchmark times,
    compared with the oracle everywhere: the flat reduce (every element),
    the tree step of rank 5 (every element of its chunk in all 8
    destinations, nothing written outside it), the quantizer (every code and
    scale of every rank), DRR-REQUANT with the fused BF16 output and the
    separate N=1 dequantization (every block). The oracle is block-local, so
    it runs over windows of whole blocks in a thread pool; the end-to-end
    error of the GPU's BF16 result D against the unquantized sum T is
    asserted on every element: |D - T| <= N 2^-3 A_b + 2^-8 |D|, with A_b the
    largest absmax of the block over the ranks and 2^-8 the unit roundoff of
    BF16's 8-bit significand (the output is rounded to BF16); the tighter
    N 2^-3 A_b + 2^-9 |D| is asserted on this message as well."""
    w = G.WORKLOADS["lp_bf16"]
    fmt, block, n, count = O.FMT[w.fp8], w.block, w.nsrc, w.count
    nb = count // block
    log("lp_bf16 generate")
    srcs = w.sources()
    log("lp_bf16 upload + gpu")
    ts = [to_gpu(x) for x in srcs]
    flat = torch.empty(count, dtype=torch.bfloat16, device=DEV)
    rx.rx_reduce_flat(ts, flat)
    k = 5
    lo5, hi5 = O.tree_chunk(count, n, O.BF16, k)
    dsts = [torch.zeros(count, dtype=torch.bfloat16, device=DEV) for _ in range(n)]
    rx.rx_reduce_scatter_chunk_bcast(ts, k, dsts)
    codes = [torch.empty(count, dtype=torch.uint8, device=DEV) for _ in range(n)]
    scales = [torch.empty(nb, dtype=torch.float32, device=DEV) for _ in range(n)]
    rx.rx_quant_fp8(ts, w.fp8, block, codes, scales)
    oc = torch.empty(count, dtype=torch.uint8, device=DEV)
    osc = torch.empty(nb, dtype=torch.float32, device=DEV)
    hp = torch.empty(count, dtype=torch.bfloat16, device=DEV)
    rx.rx_dequant_reduce_requant(codes, scales, w.fp8, block, rx.RX_DRR_REQUANT, oc, osc, hp)
    hp2 = torch.empty(count, dtype=torch.bfloat16, device=DEV)
    rx.rx_dequant_reduce_requant([oc], [osc], w.fp8, block, rx.RX_DRR_SUM, out_hp=hp2)
    sync()
    log("lp_bf16 download")
    del ts
    outside_clean = all(not d[:lo5].view(torch.int16).any().item() and
                        not d[hi5:].view(torch.int16).any().item() for d in dsts)
    g_tree = [to_host(d[lo5:hi5]) for d in dsts]
    del dsts
    g_flat = to_host(flat)
    g_codes = [c.cpu().numpy() for c in codes]
    g_scales = [q.cpu().numpy() for q in scales]
    g_oc, g_os = oc.cpu().numpy(), osc.cpu().numpy()
    g_hp, g_hp2 = to_host(hp), to_host(hp2)
    del flat, codes, scales, oc, osc, hp, hp2
    torch.cuda.empty_cache()
    assert outside_clean, "tree step wrote outside its chunk"

    win = 4096 * block                    # elements per window (whole blocks)
    u, n_f = 2.0 ** -3, float(n)

    def check(i0):
        i1 = min(i0 + win, count)
        b0, b1 = i0 // block, -(-i1 // block)
        x = [s[i0:i1] for s in srcs]
        where = f"window [{i0}, {i1})"
        r_flat = O.reduce_flat(x, O.BF16)
        if not bits_equal(g_flat[i0:i1], r_flat):
            return f"flat {where}: " + first_mismatch(g_flat[i0:i1], r_flat)
        t0, t1 = max(i0, lo5), min(i1, hi5)
        if t0 < t1:
            for j in range(n):
                got = g_tree[j][t0 - lo5:t1 - lo5]
                if not bits_equal(got, r_flat[t0 - i0:t1 - i0]):
                    return f"tree dst {j} {where}: " + first_mismatch(got, r_flat[t0 - i0:t1 - i0])
        rc, rs = O.quant_fp8(x, O.BF16, fmt, block)
        for r in range(n):
            if not bits_equal(g_codes[r][i0:i1], rc[r]):
                return f"codes rank {r} {where}: " + first_mismatch(g_codes[r][i0:i1], rc[r])
            if not bits_equal(g_scales[r][b0:b1], rs[r]):
                return f"scales rank {r} {where}: " + first_mismatch(g_scales[r][b0:b1], rs[r])
        r_oc, r_os, r_hp = O.dequant_reduce_requant(rc, rs, fmt, block, O.DRR_REQUANT, O.BF16, True)
        if not bits_equal(g_oc[i0:i1], r_oc):
            return f"requant codes {where}: " + first_mismatch(g_oc[i0:i1], r_oc)
        if not bits_equal(g_os[b0:b1], r_os):
            return f"requant scales {where}: " + first_mismatch(g_os[b0:b1], r_os)
        if not bits_equal(g_hp[i0:i1], r_hp):
            return f"fused BF16 output {where}: " + first_mismatch(g_hp[i0:i1], r_hp)
        _, _, r_hp2 = O.dequant_reduce_requant([r_oc], [r_os], fmt, block, O.DRR_SUM, O.BF16)
        if not bits_equal(g_hp2[i0:i1], r_hp2):
            return f"separate dequant {where}: " + first_mismatch(g_hp2[i0:i1], r_hp2)
        # end-to-end error of the GPU's BF16 result against the exact sum
        X = np.stack([O.bf16_to_f32(xi).astype(np.float64) for xi in x])
        T = X.sum(axis=0)
        Ab = np.repeat(np.abs(X).reshape(n, -1, block).max(axis=2).max(axis=0), block)
        D = O.bf16_to_f32(g_hp[i0:i1]).astype(np.float64)
        err = np.abs(D - T)
        bound = n_f * u * Ab + 2.0 ** -8 * np.abs(D)
        if not np.all(err <= bound):
            i = int(np.argmax(err - bound))
            return f"error bound {where}: element {i0 + i} err {err[i]} > bound {bound[i]}"
        return float(np.max(err / bound)), float(np.max(err / (n_f * u * Ab + 2.0 ** -9 * np.abs(D))))

    log(f"lp_bf16 oracle over {-(-count // win)} windows, {_pool_size()} threads")
    worst, worst9 = 0.0, 0.0
    with ThreadPoolExecutor(_pool_size()) as ex:
        for res in ex.map(check, range(0, count, win)):
            assert not isinstance(res, str), res
            worst, worst9 = max(worst, res[0]), max(worst9, res[1])
    log(f"lp_bf16 max err/bound = {worst:.4f} (with 2^-9 |D|: {worst9:.4f})")
    # the tighter form N 2^-3 A_b + 2^-9 |D| (not a bound for every input)
    # holds on this message too
    assert worst9 <= 1.0


# ---------------------------------------------------------------------------
# Hardware converters and the cross-lane maximum, swept exhaustively
# ---------------------------------------------------------------------------

CHUNK = 1 << 28


def _oracle_encode_parallel(first, n, fmt, threads=16):
    from concurrent.futures import ThreadPoolExecutor
    out = np.empty(n, np.uint8)
    per = -(-n // threads)

    def job(t):
        lo = t * per
        hi = min(n, lo + per)
        if lo < hi:
            out[lo:hi] = O.fp8_encode_bits(first + lo, hi - lo, fmt)
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(job, range(threads)))
    return out


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_fp8_encode_exhaustive(fmt):
    """All 2^32 FP32 patterns (NaNs excluded) through the kernels' clamp +
    hardware encode, against the oracle's encode."""
    out = torch.empty(CHUNK, dtype=torch.uint8, device=DEV)
    for first in range(0, 1 << 32, CHUNK):
        log(f"fp8 encode sweep fmt={fmt} first={first:#x}")
        rx.rxtest_fp8_encode_bits(first, CHUNK, FMTS[fmt], out)
        sync()
        got = out.cpu().numpy()
        ref = _oracle_encode_parallel(first, CHUNK, fmt)
        u = np.arange(CHUNK, dtype=np.uint32) + np.uint32(first)
        notnan = (u & 0x7FFFFFFF) <= 0x7F800000
        bad = np.nonzero((got != ref) & notnan)[0]
        assert bad.size == 0, f"{bad.size} mismatches, first pattern {first + bad[0]:#010x}: got {got[bad[0]]:#x} want {ref[bad[0]]:#x}"


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_block_scale_exhaustive(fmt):
    """The kernels' block scale and reciprocal (FMA-corrected quotients that
    must equal the correctly rounded FP32 divisions; degenerate blocks -> 1)
    for every non-negative FP32 block absmax A up to +inf, including zero,
    subnormals and the thresholds where A / FMAX underflows or FMAX / A
    overflows, and NaN patterns, against the oracle."""
    from concurrent.futures import ThreadPoolExecutor
    end = 0x7F800001                      # through +inf
    s_d = torch.empty(CHUNK, dtype=torch.float32, device=DEV)
    r_d = torch.empty(CHUNK, dtype=torch.float32, device=DEV)
    ranges = [(first, min(CHUNK, end - first)) for first in range(0, end, CHUNK)]
    ranges += [(0x7F800001, 4096), (0x7FC00000, 4096), (0x7FFFF000, 4096)]   # NaNs
    for first, n in ranges:
        log(f"block scale sweep fmt={fmt} first={first:#x}")
        rx.rxtest_block_scale_bits(first, n, FMTS[fmt], s_d, r_d)
        sync()
        gs, gr = s_d[:n].cpu().numpy(), r_d[:n].cpu().numpy()
        rs, rr = np.empty(n, np.float32), np.empty(n, np.float32)
        per = -(-n // 16)

        def job(t):
            lo, hi = t * per, min(n, (t + 1) * per)
            if lo < hi:
                rs[lo:hi], rr[lo:hi] = O.block_scale_bits(first + lo, hi - lo, fmt)
        with ThreadPoolExecutor(16) as ex:
            list(ex.map(job, range(16)))
        for name, g, r in (("s", gs, rs), ("r", gr, rr)):
            bad = np.nonzero(g.view(np.uint32) != r.view(np.uint32))[0]
            assert bad.size == 0, (f"{name}: {bad.size} mismatches, first A pattern "
                                   f"{first + bad[0]:#010x}: got {g[bad[0]]!r} want {r[bad[0]]!r}")


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_fp8_decode_all_codes(fmt):
    codes = torch.arange(256, dtype=torch.int32, device=DEV).to(torch.uint8)
    out = torch.empty(256, dtype=torch.float32, device=DEV)
    rx.rxtest_fp8_decode(codes, FMTS[fmt], out)
    sync()
    got = out.cpu().numpy()
    ref = O.fp8_decode(np.arange(256, dtype=np.uint8), fmt)
    ok = ~np.isnan(ref)
    assert np.array_equal(np.isnan(got), ~ok)
    assert bits_equal(got[ok], ref[ok])


def test_bf16_round_exhaustive():
    from concurrent.futures import ThreadPoolExecutor
    out = torch.empty(CHUNK, dtype=torch.bfloat16, device=DEV)
    for first in range(0, 1 << 32, CHUNK):
        log(f"bf16 sweep first={first:#x}")
        rx.rxtest_bf16_round_bits(first, CHUNK, out)
        sync()
        got = to_host(out)
        x = (np.arange(CHUNK, dtype=np.uint32) + np.uint32(first)).view(np.float32)
        ref = np.empty(CHUNK, np.uint16)
        per = CHUNK // 16

        def job(t):
            ref[t * per:(t + 1) * per] = O.f32_to_bf16(x[t * per:(t + 1) * per])
        with ThreadPoolExecutor(16) as ex:
            list(ex.map(job, range(16)))
        notnan = ~np.isnan(x)
        bad = np.nonzero((got != ref) & notnan)[0]
        assert bad.size == 0, f"{bad.size} mismatches, first pattern {first + bad[0]:#010x}"


def test_group_max_lane_layout():
    rng = np.random.default_rng(17)
    vals = rng.integers(0, 2 ** 31, size=64 * 64, dtype=np.uint32)
    t = torch.from_numpy(vals.view(np.int32)).to(DEV)
    out = torch.empty_like(t)
    for g in (1, 2, 4, 8, 16, 32, 64):
        rx.rxtest_group_max(t, g, out)
        sync()
        got = out.cpu().numpy().view(np.uint32)
        ref = np.repeat(vals.reshape(-1, g).max(axis=1), g)
        assert np.array_equal(got, ref), f"g={g}"


# ---------------------------------------------------------------------------
# Launch-shape thresholds
# ---------------------------------------------------------------------------

# Counts at and beside the size thresholds at which the launchers change
# kernel, tile or workgroups per CU on a 256-CU MI355X (on another device the
# cases still hold, at other launch shapes): every side must give the
# oracle's bits.
_BOUNDARY_CASES = [
    # flat reduce: decode-size below 131,072 16-byte vectors
    ("flat", O.FP32, 8, (1 << 19) - 1), ("flat", O.FP32, 8, 1 << 19), ("flat", O.FP32, 8, (1 << 19) + 1),
    ("flat", O.BF16, 3, (1 << 20) - 1), ("flat", O.BF16, 3, (1 << 20) + 1),
    ("flat", O.BF16, 8, (1 << 20) + 1), ("flat", O.FP32, 13, (1 << 19) + 3),
    # flat reduce: medium up to 16 whole tiles per CU (4096 tiles of 256
    # vectors), large above
    ("flat", O.BF16, 8, (1 << 23) + 3), ("flat", O.BF16, 8, (1 << 23) + 2048 + 1),
    ("flat", O.FP32, 5, (1 << 22) + 1), ("flat", O.FP32, 5, (1 << 22) + 1024 + 3),
    ("flat", O.BF16, 6, (1 << 20) - 8 + 1), ("flat", O.BF16, 2, (1 << 20) + 2048 * 3 + 7),
    # quantizer, 8 FP32 sources: decode-size below 2,048 tiles of 1024,
    # four workgroups per CU below 16,384, two above
    ("quant", O.FP32, 8, 255 * 1024), ("quant", O.FP32, 8, 255 * 1024 + 1), ("quant", O.FP32, 8, 256 * 1024),
    ("quant", O.FP32, 8, 2047 * 1024), ("quant", O.FP32, 8, 2047 * 1024 + 1), ("quant", O.BF16, 8, 2048 * 1024 + 7),
    # whole decode-size tiles: the loop-free kernel up to 16 (BF16) or 8
    # (FP32) large tiles per CU, the large kernels above and for ragged counts
    ("quant", O.BF16, 8, 1 << 20), ("quant", O.BF16, 8, (1 << 20) + 512), ("quant", O.BF16, 8, (1 << 20) - 509),
    ("quant", O.FP32, 8, 288 * 1024),
    # DRR: decode-size below 1,024 tiles of 1024 codes; codes only: four
    # workgroups per CU below 8,192 tiles
    ("drr", O.FP32, 8, 1023 * 1024), ("drr", O.FP32, 8, 1023 * 1024 + 1), ("drr", O.FP32, 8, 1024 * 1024 + 5),
    ("drr", O.FP32, 8, 8191 * 1024 - 5), ("drr", O.FP32, 8, 8192 * 1024 + 3),
    # one-pass LP allreduce: BF16 8-byte lanes up to 2,048 tiles of 512,
    # 256-thread workgroups up to 4,096 tiles (FP32: tiles of 256)
    ("lp", O.BF16, 8, 512 * 512), ("lp", O.BF16, 8, 512 * 512 + 1), ("lp", O.BF16, 8, 4096 * 512 + 1),
    ("lp", O.BF16, 8, 2048 * 512), ("lp", O.BF16, 8, 2048 * 512 - 3), ("lp", O.BF16, 8, 2048 * 512 + 1),
    ("lp", O.FP32, 8, 4096 * 256), ("lp", O.FP32, 8, 4096 * 256 + 1),
]


@pytest.mark.parametrize("what,dtype,n,count", _BOUNDARY_CASES)
def test_launch_policy_boundaries(what, dtype, n, count):
    fmt, block = (O.E4M3, 128) if dtype == O.FP32 else (O.E5M2, 256)
    log(f"boundary {what} dtype={dtype} n={n} count={count}")
    srcs = [G.fill(count, dtype, G.NORMAL_OUTLIER, seed=9500 + r + count % 101, rank=r) for r in range(n)]
    if what == "flat":
        g = Guarded(count, TD[dtype])
        rx.rx_reduce_flat([to_gpu(x) for x in srcs], g.t)
        sync()
        ref = O.reduce_flat(srcs, dtype)
        got = to_host(g.t)
        assert bits_equal(got, ref), first_mismatch(got, ref)
        assert g.guards_intact()
    elif what == "quant":
        gc, gs = _quant_gpu(srcs, dtype, fmt, block, count)
        rc, rs = O.quant_fp8(srcs, dtype, fmt, block)
        for j in range(n):
            assert bits_equal(gc[j], rc[j]), f"codes src={j}: " + first_mismatch(gc[j], rc[j])
            assert bits_equal(gs[j], rs[j]), f"scales src={j}: " + first_mismatch(gs[j], rs[j])
    elif what == "drr":
        codes, scales = O.quant_fp8(srcs, dtype, fmt, block)
        cases = ((codes, scales, O.DRR_REQUANT, O.FP32, False),      # codes only (16 x 1)
                 (codes, scales, O.DRR_REQUANT, O.BF16, True),       # several sources: staged
                 (codes[:1], scales[:1], O.DRR_SUM, O.FP32, True),   # one source, FP32 (4 x 4)
                 (codes[:1], scales[:1], O.DRR_SUM, O.BF16, True))   # one source, BF16 (8 x 2)
        for cs_, ss_, mode, hp_dtype, want_hp in cases:
            got = _drr_gpu(cs_, ss_, fmt, block, mode, hp_dtype, want_hp, count)
            ref = O.dequant_reduce_requant(cs_, ss_, fmt, block, mode, hp_dtype, want_hp)
            for name, g_, r_ in zip(("codes", "scales", "hp"), got, ref):
                assert (g_ is None) == (r_ is None)
                if g_ is not None:
                    assert bits_equal(g_, r_), f"mode={mode} n={len(cs_)} {name}: " + first_mismatch(g_, r_)
    else:
        ts = [to_gpu(x) for x in srcs]
        ws = torch.empty(rx.rx_allreduce_local_workspace(n, count, block), dtype=torch.uint8, device=DEV)
        rx.rx_allreduce_local(ts, rx.RX_ALGO_LOWPREC, FMTS[fmt], block, ws)
        sync()
        ref = [x.copy() for x in srcs]
        O.allreduce_local(ref, dtype, O.ALGO_LOWPREC, fmt, block)
        for j in range(n):
            got = to_host(ts[j])
            assert bits_equal(got, ref[j]), f"rank={j}: " + first_mismatch(got, ref[j])


# ---------------------------------------------------------------------------
# HIP graphs and concurrent streams
# ---------------------------------------------------------------------------

def _lp_all(ts, fmt, block, n, count):
    nb = -(-count // block)
    dt = ts[0].dtype
    out = dict(
        flat=torch.empty(count, dtype=dt, device=DEV),
        tree=[torch.empty(count, dtype=dt, device=DEV) for _ in range(n)],
        codes=[torch.empty(count, dtype=torch.uint8, device=DEV) for _ in range(n)],
        scales=[torch.empty(nb, dtype=torch.float32, device=DEV) for _ in range(n)],
        oc=torch.empty(count, dtype=torch.uint8, device=DEV),
        osc=torch.empty(nb, dtype=torch.float32, device=DEV),
        hp=torch.empty(count, dtype=dt, device=DEV),
        lpc=[torch.empty(count, dtype=torch.uint8, device=DEV) for _ in range(n)],
        lps=[torch.empty(nb, dtype=torch.float32, device=DEV) for _ in range(n)],
        oc2=torch.empty(count, dtype=torch.uint8, device=DEV),
        osc2=torch.empty(nb, dtype=torch.float32, device=DEV),
    )

    def run():
        rx.rx_reduce_flat(ts, out["flat"])
        rx.rx_reduce_scatter_chunk_bcast(ts, 1, out["tree"])
        rx.rx_quant_fp8(ts, fmt, block, out["codes"], out["scales"])
        rx.rx_dequant_reduce_requant(out["codes"], out["scales"], fmt, block, rx.RX_DRR_REQUANT,
                                     out["oc"], out["osc"], out["hp"])
        rx.rx_lp_reduce_scatter_chunk_bcast(out["codes"], out["scales"], fmt, block, 2,
                                            out["lpc"], out["lps"])
        rx.rx_dequant_reduce_requant(out["codes"], out["scales"], fmt, block, rx.RX_DRR_REQUANT,
                                     out["oc2"], out["osc2"])
    return out, run


def _snapshot(out):
    flat = lambda v: [v] if torch.is_tensor(v) else list(v)
    return {k: [to_host(t).copy() for t in flat(v)] for k, v in out.items()}


@pytest.mark.parametrize("count,dtype", [(262_144, G.BF16), (3 * (1 << 20) + 77, G.BF16),
                                         (3 * (1 << 20) + 77, G.FP32)])
def test_graph_replays_match_eager(count, dtype):
    """All five entry points captured in one HIP graph (no memset nodes: the
    library enqueues kernels only; large ragged messages take two launches
    in the quantizer, the FP32 flat reduce and DRR), replayed three times
    with new inputs written eagerly between replays; every replay must equal
    an eager run on the same inputs."""
    n = 8
    fmt, block = ("e5m2", 256) if dtype == G.BF16 else ("e4m3", 128)
    inputs = [[to_gpu(G.fill(count, dtype, G.NORMAL, seed=6000 + 10 * k + count % 7, rank=r))
               for r in range(n)] for k in range(3)]
    ts = [torch.empty(count, dtype=TD[dtype], device=DEV) for _ in range(n)]
    out, run = _lp_all(ts, fmt, block, n, count)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    def clear():   # the chunk steps leave everything outside their chunk as it was
        for v in out.values():
            for t in ([v] if torch.is_tensor(v) else v):
                t.zero_()

    for k in range(3):
        log(f"graph replay {k} count={count} dtype={dtype}")
        for t, x in zip(ts, inputs[k]):
            t.copy_(x)
        clear()
        sync()
        g.replay()
        sync()
        got = _snapshot(out)
        clear()
        run()
        sync()
        ref = _snapshot(out)
        for key in got:
            for a, b in zip(got[key], ref[key]):
                assert bits_equal(a, b), f"replay {k} {key}: " + first_mismatch(a, b)


def test_concurrent_streams_are_independent():
    """Calls on two streams at once (the library keeps no state) give the
    same results as the same calls one after the other."""
    n, fmt, block, count = 8, "e4m3", 128, 2 * (1 << 20) + 3
    ins = [[to_gpu(G.fill(count, G.FP32, G.NORMAL_OUTLIER, seed=7000 + s, rank=r)) for r in range(n)]
           for s in range(2)]
    outs, runs = zip(*[_lp_all(ins[s], fmt, block, n, count) for s in range(2)])
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    cur = torch.cuda.current_stream()
    for s in range(2):
        streams[s].wait_stream(cur)
    for _ in range(3):
        for s in range(2):
            with torch.cuda.stream(streams[s]):
                runs[s]()
    for s in range(2):
        cur.wait_stream(streams[s])
    sync()
    got = [_snapshot(o) for o in outs]
    for s in range(2):
        runs[s]()
        sync()
        ref = _snapshot(outs[s])
        for key in ref:
            for a, b in zip(got[s][key], ref[key]):
                assert bits_equal(a, b), f"stream {s} {key}: " + first_mismatch(a, b)


# ---------------------------------------------------------------------------
# Local allreduce dispatcher and in-place low-precision tree step
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [O.FP32, O.BF16])
@pytest.mark.parametrize("algo", [rx.RX_ALGO_FLAT, rx.RX_ALGO_TREE, rx.RX_ALGO_LOWPREC])
def test_allreduce_local(dtype, algo):
    n = 8
    fmt, block = (O.E4M3, 128) if dtype == O.FP32 else (O.E5M2, 256)
    for count in [1, 1000, 262_144, 3 * (1 << 20) + 5]:
        log(f"allreduce_local algo={algo} dtype={dtype} count={count}")
        srcs = [G.fill(count, dtype, G.NORMAL_OUTLIER, seed=8000 + count % 97, rank=r) for r in range(n)]
        ts = [to_gpu(s) for s in srcs]
        ws = torch.empty(rx.rx_allreduce_local_workspace(n, count, block), dtype=torch.uint8, device=DEV)
        rx.rx_allreduce_local(ts, algo, FMTS[fmt], block, ws)
        sync()
        ref = [s.copy() for s in srcs]
        O.allreduce_local(ref, dtype, {rx.RX_ALGO_FLAT: O.ALGO_FLAT, rx.RX_ALGO_TREE: O.ALGO_TREE,
                                       rx.RX_ALGO_LOWPREC: O.ALGO_LOWPREC}[algo], fmt, block)
        for j in range(n):
            got = to_host(ts[j])
            assert bits_equal(got, ref[j]), f"count={count} rank={j}: " + first_mismatch(got, ref[j])


@pytest.mark.parametrize("dtype", [O.FP32, O.BF16])
@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_allreduce_local_lowprec_every_block(dtype, fmt):
    """The low-precision allreduce for every block size: blocks of at most 64
    16-byte vectors run the one-pass kernel (codes in registers), larger ones
    quantize into the workspace first; ragged counts, 1..16 ranks, and a rank
    of zeros (degenerate blocks, s = r = 1). On a 256-CU MI355X the counts
    reach every launch shape of the one-pass kernel: 8-byte lanes (BF16, up
    to 512 tiles of 64 16-byte vectors; one tile per wave without a loop
    when the count is whole tiles), 256-thread workgroups (up to 4096
    tiles) and the grid-stride launch above."""
    for block in (32, 64, 128, 256, 512, 1024):
        for n, count in ((8, 70001), (3, 4096 + 17), (16, 1000), (1, 513), (4, 300_005),
                         (8, (1 << 20) + 77), (8, 65536)):
            log(f"allreduce_local lowprec dtype={dtype} fmt={fmt} block={block} n={n} count={count}")
            srcs = [G.fill(count, dtype, G.NORMAL_OUTLIER, seed=9100 + block + n, rank=r)
                    for r in range(n)]
            if n == 3:
                srcs[1][:] = 0
            ts = [to_gpu(x) for x in srcs]
            ws = torch.empty(rx.rx_allreduce_local_workspace(n, count, block), dtype=torch.uint8,
                             device=DEV)
            rx.rx_allreduce_local(ts, rx.RX_ALGO_LOWPREC, FMTS[fmt], block, ws)
            sync()
            ref = [x.copy() for x in srcs]
            O.allreduce_local(ref, dtype, O.ALGO_LOWPREC, fmt, block)
            for j in range(n):
                got = to_host(ts[j])
                assert bits_equal(got, ref[j]), (f"block={block} n={n} rank={j}: "
                                                 + first_mismatch(got, ref[j]))


@pytest.mark.parametrize("n", [1, 3, 16])
def test_allreduce_local_rank_counts(n):
    """Every algorithm with other rank counts, ragged length."""
    count = 4133
    for dtype in (O.FP32, O.BF16):
        fmt, block = (O.E4M3, 64) if dtype == O.FP32 else (O.E5M2, 512)
        srcs = [G.fill(count, dtype, G.NORMAL, seed=8300 + n, rank=r) for r in range(n)]
        for algo, oalgo in ((rx.RX_ALGO_FLAT, O.ALGO_FLAT), (rx.RX_ALGO_TREE, O.ALGO_TREE),
                            (rx.RX_ALGO_LOWPREC, O.ALGO_LOWPREC)):
            log(f"allreduce_local n={n} dtype={dtype} algo={algo}")
            ts = [to_gpu(s) for s in srcs]
            ws = torch.empty(rx.rx_allreduce_local_workspace(n, count, block), dtype=torch.uint8,
                             device=DEV)
            rx.rx_allreduce_local(ts, algo, FMTS[fmt], block, ws)
            sync()
            ref = [s.copy() for s in srcs]
            O.allreduce_local(ref, dtype, oalgo, fmt, block)
            for j in range(n):
                got = to_host(ts[j])
                assert bits_equal(got, ref[j]), f"algo={algo} rank={j}: " + first_mismatch(got, ref[j])


def test_allreduce_local_rank_id_example():
    for algo in (rx.RX_ALGO_FLAT, rx.RX_ALGO_TREE, rx.RX_ALGO_LOWPREC, rx.RX_ALGO_AUTO):
        ts = [torch.full((10, 20), float(r), dtype=torch.float32, device=DEV) for r in range(8)]
        ws = torch.empty(rx.rx_allreduce_local_workspace(8, 200, 128), dtype=torch.uint8, device=DEV)
        rx.rx_allreduce_local(ts, algo, "e4m3", 128, ws)
        sync()
        assert all(torch.all(t == 28.0).item() for t in ts), f"algo {algo}"


def test_allreduce_local_auto_switch(monkeypatch):
    """AUTO takes the low-precision path only with RX_LOW_PRECISION_ENABLE=1
    and messages of at least 16 MiB; otherwise the flat pass."""
    n, count, fmt, block = 8, 8 * (1 << 20) + 3, "e5m2", 256   # BF16: 16 MiB + 6 bytes
    srcs = [G.fill(count, G.BF16, G.LAPLACE, seed=8500, rank=r) for r in range(n)]
    ws = torch.empty(rx.rx_allreduce_local_workspace(n, count, block), dtype=torch.uint8, device=DEV)
    for env, algo in (("0", O.ALGO_FLAT), ("1", O.ALGO_LOWPREC)):
        monkeypatch.setenv("RX_LOW_PRECISION_ENABLE", env)
        log(f"allreduce_local auto env={env}")
        ts = [to_gpu(s) for s in srcs]
        rx.rx_allreduce_local(ts, rx.RX_ALGO_AUTO, fmt, block, ws)
        sync()
        ref = [s.copy() for s in srcs]
        O.allreduce_local(ref, O.BF16, algo, O.E5M2, block)
        for j in (0, n - 1):
            got = to_host(ts[j])
            assert bits_equal(got, ref[j]), f"env={env} rank={j}: " + first_mismatch(got, ref[j])
    # below 16 MiB the switch does not apply
    monkeypatch.setenv("RX_LOW_PRECISION_ENABLE", "1")
    small = [s[:1000].copy() for s in srcs]
    ts = [to_gpu(s) for s in small]
    rx.rx_allreduce_local(ts, rx.RX_ALGO_AUTO, fmt, block, None)
    sync()
    ref = [s.copy() for s in small]
    O.allreduce_local(ref, O.BF16, O.ALGO_FLAT)
    assert bits_equal(to_host(ts[0]), ref[0])


@pytest.mark.parametrize("count", [20_000, 3 * (1 << 20) + 5])
def test_lp_tree_in_place(count):
    n, fmt, block = 8, O.E4M3, 128
    srcs = [G.fill(count, O.FP32, G.NORMAL, seed=9000 + count % 13, rank=r) for r in range(n)]
    codes, scales = O.quant_fp8(srcs, O.FP32, fmt, block)
    tc = [to_gpu(c) for c in codes]
    tsc = [to_gpu(s) for s in scales]
    ref_c = [c.copy() for c in codes]
    ref_s = [s.copy() for s in scales]
    for k in range(n):
        log(f"lp tree in place count={count} rank={k}")
        rx.rx_lp_reduce_scatter_chunk_bcast(tc, tsc, FMTS[fmt], block, k, tc, tsc)
        sync()
        O.lp_reduce_scatter_chunk_bcast([c.copy() for c in ref_c], [s.copy() for s in ref_s],
                                        fmt, block, k, ref_c, ref_s)
    for j in range(n):
        assert bits_equal(to_host(tc[j]), ref_c[j]) and bits_equal(to_host(tsc[j]), ref_s[j])


# ---------------------------------------------------------------------------
# Launch-shape independence: the decode-size and large-message kernels (and
# their different grids) give the same bits on the same data
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [O.FP32, O.BF16])
def test_paths_agree_across_launch_shapes(dtype):
    n, big, small = 8, 1 << 22, 1 << 17      # large-message vs decode-size launches
    log(f"launch-shape independence dtype={dtype}")
    srcs = [to_gpu(G.fill(big, dtype, G.NORMAL, seed=7100 + dtype, rank=r)) for r in range(n)]
    td = TD[dtype]
    # flat reduce
    yb = torch.empty(big, dtype=td, device=DEV)
    ys = torch.empty(small, dtype=td, device=DEV)
    rx.rx_reduce_flat(srcs, yb)
    rx.rx_reduce_flat(srcs, ys, count=small)
    # in-place flat allreduce (tree kernels over the whole range)
    ab = [s.clone() for s in srcs]
    as_ = [s[:small].clone() for s in srcs]
    rx.rx_allreduce_local(ab, rx.RX_ALGO_FLAT)
    rx.rx_allreduce_local(as_, rx.RX_ALGO_FLAT)
    # quantizer and DRR with the high-precision output
    for fmt, block in ((O.E4M3, 128), (O.E5M2, 256)):
        f = FMTS[fmt]
        cb = [torch.empty(big, dtype=torch.uint8, device=DEV) for _ in range(n)]
        sb = [torch.empty(big // block, dtype=torch.float32, device=DEV) for _ in range(n)]
        cs = [torch.empty(small, dtype=torch.uint8, device=DEV) for _ in range(n)]
        ss = [torch.empty(small // block, dtype=torch.float32, device=DEV) for _ in range(n)]
        rx.rx_quant_fp8(srcs, f, block, cb, sb)
        rx.rx_quant_fp8(srcs, f, block, cs, ss, count=small)
        ob, osb, hb = (torch.empty(big, dtype=torch.uint8, device=DEV),
                       torch.empty(big // block, dtype=torch.float32, device=DEV),
                       torch.empty(big, dtype=td, device=DEV))
        os1, oss, hs = (torch.empty(small, dtype=torch.uint8, device=DEV),
                        torch.empty(small // block, dtype=torch.float32, device=DEV),
                        torch.empty(small, dtype=td, device=DEV))
        rx.rx_dequant_reduce_requant(cb, sb, f, block, rx.RX_DRR_REQUANT, ob, osb, hb)
        rx.rx_dequant_reduce_requant(cs, ss, f, block, rx.RX_DRR_REQUANT, os1, oss, hs, count=small)
        sync()
        for j in range(n):
            assert torch.equal(cb[j][:small], cs[j]) and torch.equal(
                sb[j][:small // block].view(torch.int32), ss[j].view(torch.int32)), f"quant {fmt} src {j}"
        assert torch.equal(ob[:small], os1)
        assert torch.equal(osb[:small // block].view(torch.int32), oss.view(torch.int32))
        iv = torch.int16 if dtype == O.BF16 else torch.int32
        assert torch.equal(hb[:small].view(iv), hs.view(iv)), f"drr hp {fmt}"
    sync()
    iv = torch.int16 if dtype == O.BF16 else torch.int32
    assert torch.equal(yb[:small].view(iv), ys.view(iv)), "flat"
    for j in range(n):
        assert torch.equal(ab[j][:small].view(iv), as_[j].view(iv)), f"allreduce buffer {j}"


@pytest.mark.parametrize("n", list(range(1, 17)))
def test_every_source_count(n):
    """Every source count 1..16 (each is its own kernel instance) through
    every entry point on ragged decode-size messages, every rank of both
    tree steps included; the flat reduce also above the decode-size
    threshold (the tiled kernel)."""
    algos = ((rx.RX_ALGO_FLAT, O.ALGO_FLAT), (rx.RX_ALGO_TREE, O.ALGO_TREE),
             (rx.RX_ALGO_LOWPREC, O.ALGO_LOWPREC))
    for dtype in (O.FP32, O.BF16):
        fmt, block = (O.E4M3, 128) if dtype == O.FP32 else (O.E5M2, 256)
        for count in (1003, 37_777):
            srcs = [G.fill(count, dtype, G.NORMAL_OUTLIER, seed=9000 + 7 * n + count % 13, rank=r)
                    for r in range(n)]
            log(f"every-n n={n} dtype={dtype} count={count}: flat, tree (all ranks)")
            g = Guarded(count, TD[dtype])
            rx.rx_reduce_flat([to_gpu(x) for x in srcs], g.t)
            sync()
            ref = O.reduce_flat(srcs, dtype)
            got = to_host(g.t)
            assert bits_equal(got, ref), "flat: " + first_mismatch(got, ref)
            assert g.guards_intact()
            for k in range(n):
                _tree_case(srcs, dtype, count, k)

            log(f"every-n n={n} dtype={dtype} count={count}: quant, dequant-reduce-requant")
            gc, gs = _quant_gpu(srcs, dtype, fmt, block, count)
            rc, rs = O.quant_fp8(srcs, dtype, fmt, block)
            for j in range(n):
                assert bits_equal(gc[j], rc[j]), f"codes src={j}: " + first_mismatch(gc[j], rc[j])
                assert bits_equal(gs[j], rs[j]), f"scales src={j}: " + first_mismatch(gs[j], rs[j])
            for mode, hp_dtype, want_hp in ((O.DRR_SUM, dtype, True), (O.DRR_REQUANT, dtype, True),
                                            (O.DRR_REQUANT, O.FP32, False)):
                got = _drr_gpu(rc, rs, fmt, block, mode, hp_dtype, want_hp, count)
                ref = O.dequant_reduce_requant(rc, rs, fmt, block, mode, hp_dtype, want_hp)
                for name, a, b in zip(("codes", "scales", "hp"), got, ref):
                    assert (a is None) == (b is None)
                    if a is not None:
                        assert bits_equal(a, b), f"drr mode={mode} {name}: " + first_mismatch(a, b)

            log(f"every-n n={n} dtype={dtype} count={count}: low-precision tree (all ranks), allreduce")
            for k in range(n):
                _lp_tree_case(rc, rs, fmt, block, k, count, hp_dtype=(dtype, None)[k % 2])
            for algo, oalgo in algos:
                ts = [to_gpu(x) for x in srcs]
                ws = torch.empty(max(1, rx.rx_allreduce_local_workspace(n, count, block)),
                                 dtype=torch.uint8, device=DEV)
                rx.rx_allreduce_local(ts, algo, FMTS[fmt], block, ws)
                sync()
                ref = [x.copy() for x in srcs]
                O.allreduce_local(ref, dtype, oalgo, fmt, block)
                for j in range(n):
                    got = to_host(ts[j])
                    assert bits_equal(got, ref[j]), f"allreduce algo={algo} rank={j}: " + first_mismatch(got, ref[j])

    # above the decode-size threshold: the tiled flat kernel, ragged end
    count = (1 << 20) + 4101
    for dtype in (O.FP32, O.BF16):
        log(f"every-n n={n} dtype={dtype} count={count}: flat (tiled)")
        srcs = [G.fill(count, dtype, G.NORMAL, seed=9500 + n, rank=r) for r in range(n)]
        g = Guarded(count, TD[dtype])
        rx.rx_reduce_flat([to_gpu(x) for x in srcs], g.t)
        sync()
        ref = O.reduce_flat(srcs, dtype)
        got = to_host(g.t)
        assert bits_equal(got, ref), "flat tiled: " + first_mismatch(got, ref)
        assert g.guards_intact()


def test_debug_env_logs_launches():
    """RX_DEBUG=1 prints every launch's kernel and grid (read once per
    process, so checked in a child process)."""
    import os
    import subprocess
    import sys
    log("RX_DEBUG launch log (child process)")
    code = ("import torch, allreduce_reduction_rx_amd as rx\n"
            "s = [torch.ones(1 << 12, device='cuda') for _ in range(3)]\n"
            "d = torch.empty(1 << 12, device='cuda')\n"
            "rx.rx_reduce_flat(s, d)\n"
            "torch.cuda.synchronize()\n"
            "assert torch.all(d == 3).item()\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, RX_DEBUG="1", PYTHONPATH=root + os.pathsep + os.environ.get("PYTHONPATH", ""))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       timeout=240, cwd=root)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "librx: k_reduce_flat grid" in r.stderr
