"""rx_allreduce_local_noalloc (the allocation-free variant of
rx_allreduce_local, for callers that cannot allocate) against
rx_allreduce_local with a caller workspace, through the C ABI: bit for bit,
for every algorithm, on two calls in a row, the second with a smaller input
(the scratch keeps the first call's contents). Blocks of 1024 take the
two-pass low-precision form, whose codes and scales live in the scratch;
blocks of 128 / 256 the one-pass form."""
import numpy as np
import pytest
import torch

import allreduce_reduction_rx_amd as rx
import rxgen as G
from gpu_util import DEV, log

pytestmark = pytest.mark.gpu


def _bufs(count, dtype, seed, n):
    tdt = torch.bfloat16 if dtype == G.BF16 else torch.float32
    out = []
    for r in range(n):
        h = G.fill(count, dtype, G.NORMAL_OUTLIER, seed=seed, rank=r)
        t = torch.from_numpy(h.view(np.int16) if h.dtype == np.uint16 else h).to(DEV)
        out.append(t.view(tdt) if h.dtype == np.uint16 else t)
    return out


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("dtype,fmt,block", [(G.FP32, "e4m3", 1024), (G.BF16, "e5m2", 1024),
                                             (G.FP32, "e4m3", 128), (G.BF16, "e5m2", 256)])
@pytest.mark.parametrize("algo", [rx.RX_ALGO_LOWPREC, rx.RX_ALGO_FLAT, rx.RX_ALGO_TREE])
def test_noalloc_matches_workspace_variant(dtype, fmt, block, algo):
    n = 8
    # the first call fills almost all of the scratch (low precision), the
    # second is smaller and ragged
    for count, seed in ((8_000_000, 61), (70_001, 62)):
        log(f"noalloc dtype={dtype} fmt={fmt} block={block} algo={algo} count={count}")
        a = _bufs(count, dtype, seed, n)
        b = [t.clone() for t in a]
        ws = torch.empty(rx.rx_allreduce_local_workspace(n, count, block), dtype=torch.uint8,
                         device=DEV)
        rx.rx_allreduce_local(a, algo, fmt, block, ws)
        rx.rx_allreduce_local_noalloc(b, algo, fmt, block)
        torch.cuda.synchronize()
        for j in range(n):
            assert torch.equal(_bits(a[j]), _bits(b[j])), f"rank {j}"
        del a, b, ws


def test_noalloc_oversize_rejected_and_nothing_written():
    n, count = 8, 8_355_841          # one element beyond the scratch (blocks of 1024)
    bufs = [torch.full((count,), 1.5, dtype=torch.float32, device=DEV) for _ in range(n)]
    with pytest.raises(rx.RxError) as e:
        rx.rx_allreduce_local_noalloc(bufs, rx.RX_ALGO_LOWPREC, "e4m3", 1024)
    assert e.value.status == rx.RX_ERR_SCRATCH
    torch.cuda.synchronize()
    assert all(bool((t == 1.5).all()) for t in bufs)
