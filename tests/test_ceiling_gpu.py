"""GPU checks of the streaming ceiling kernels the benchmark measures the HBM
ceilings with: the read kernel really reads every byte (its XOR sink equals
the XOR of the input), the write kernel writes exactly the pattern over
exactly the range, and the copy kernel copies exactly the range. Ragged
sizes leave a partial wave tile at the end."""
import numpy as np
import pytest
import torch

import allreduce_reduction_rx_amd as rx
from gpu_util import DEV, Guarded, log

pytestmark = pytest.mark.gpu

SIZES = [16, 4096, 4096 + 16, 65536 * 16 + 48, (3 << 20) + 1024 + 16]
PATTERN = np.array([1.0, 2.0, 3.0, 4.0], dtype=np.float32).view(np.uint8)


def random_bytes(nbytes, seed):
    g = np.random.default_rng(seed)
    return g.integers(0, 256, nbytes, dtype=np.uint8)


@pytest.mark.parametrize("nbytes", SIZES)
@pytest.mark.parametrize("wgs,nt", [(1, False), (8, True), (2, True)])
def test_stream_read_copy_write(nbytes, wgs, nt):
    log(f"ceiling kernels bytes={nbytes} wgs={wgs} nt={nt}")
    host = random_bytes(nbytes, nbytes + wgs)
    src = torch.from_numpy(host).to(DEV)

    # read: XOR of the per-thread sinks == XOR of the input's 16-byte words
    sink_bytes = rx.rxtest_stream_sink_bytes(wgs)
    sink = torch.zeros(sink_bytes, dtype=torch.uint8, device=DEV)
    rx.rxtest_stream(rx.RXTEST_READ, src, sink, nbytes, wgs, nt)
    # copy
    cp = Guarded(nbytes, torch.uint8)
    rx.rxtest_stream(rx.RXTEST_COPY, src, cp.t, nbytes, wgs, nt)
    # write
    wr = Guarded(nbytes, torch.uint8)
    rx.rxtest_stream(rx.RXTEST_WRITE, None, wr.t, nbytes, wgs, nt)
    torch.cuda.synchronize()

    want = np.bitwise_xor.reduce(host.view(np.uint32).reshape(-1, 4), axis=0)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32).reshape(-1, 4), axis=0)
    assert np.array_equal(got, want)
    assert np.array_equal(cp.t.cpu().numpy(), host) and cp.guards_intact()
    assert np.array_equal(wr.t.cpu().numpy(), np.tile(PATTERN, nbytes // 16)) and wr.guards_intact()


def test_stream_empty_launch_touches_nothing():
    log("ceiling kernels: empty launch")
    g = Guarded(4096, torch.uint8)
    before = g.t.clone()
    rx.rxtest_stream(rx.RXTEST_EMPTY, None, g.t, 4096, 4, False)
    rx.rxtest_stream(rx.RXTEST_EMPTY, None, None, 0, 1, False)
    torch.cuda.synchronize()
    assert torch.equal(g.t, before) and g.guards_intact()


@pytest.mark.parametrize("nbytes", SIZES)
@pytest.mark.parametrize("wgs,nt,pf", [(1, False, False), (4, True, False), (1, True, True), (2, False, True)])
def test_stream_mixed(nbytes, wgs, nt, pf):
    """Mixed read/write ceilings: reduce over 1, 3, 8 and 16 sources (XOR of
    the sources, 16-byte word by word) and the 2:1 / 4:1 narrowing folds,
    exactly over the range (guard bands intact), with and without the
    next-tile prefetch."""
    log(f"mixed ceiling kernels bytes={nbytes} wgs={wgs} nt={nt} prefetch={pf}")
    hosts = [random_bytes(nbytes, 7 * nbytes + r) for r in range(16)]
    srcs = [torch.from_numpy(h).to(DEV) for h in hosts]
    for nsrc in (1, 3, 8, 16):
        out = Guarded(nbytes, torch.uint8)
        rx.rxtest_stream_mixed(rx.RXTEST_MIXED_REDUCE, srcs[:nsrc], out.t, nbytes, wgs, nt, pf)
        torch.cuda.synchronize()
        want = np.bitwise_xor.reduce(np.stack(hosts[:nsrc]), axis=0)
        assert np.array_equal(out.t.cpu().numpy(), want), f"reduce nsrc={nsrc}"
        assert out.guards_intact()
    words = hosts[0].view(np.uint32).reshape(-1, 4)
    for kind, k in ((rx.RXTEST_MIXED_NARROW2, 2), (rx.RXTEST_MIXED_NARROW4, 4)):
        out = Guarded(nbytes // k, torch.uint8)
        rx.rxtest_stream_mixed(kind, srcs[:1], out.t, nbytes, wgs, nt, pf)
        torch.cuda.synchronize()
        if k == 2:
            want = np.stack([words[:, 0] ^ words[:, 1], words[:, 2] ^ words[:, 3]], axis=1)
        else:
            want = words[:, 0] ^ words[:, 1] ^ words[:, 2] ^ words[:, 3]
        assert np.array_equal(out.t.cpu().numpy(), want.astype(np.uint32).ravel().view(np.uint8)), k
        assert out.guards_intact()


@pytest.mark.parametrize("n", [1, 3, 8, 16])
@pytest.mark.parametrize("lanes,wg", [(1, 64), (2, 64), (1, 256), (2, 128)])
def test_copy_streams(n, lanes, wg):
    """The tree step's memory pattern without arithmetic: each stream's byte
    range copied into its own destination, nothing else written."""
    total = (1 << 20) + 4096
    for off, nbytes in ((0, 16), (4096, 65536 * 16), (48, (1 << 20) - 64), (16, total - 32)):
        log(f"copy streams n={n} lanes={lanes} wg={wg} off={off} bytes={nbytes}")
        hosts = [random_bytes(total, 1000 * n + 17 * off + r) for r in range(n)]
        srcs = [torch.from_numpy(h).to(DEV) for h in hosts]
        dsts = [Guarded(total, torch.uint8) for _ in range(n)]
        before = [d.t.clone() for d in dsts]
        rx.rxtest_copy_streams(srcs, [d.t for d in dsts], off, nbytes, lanes, wg)
        torch.cuda.synchronize()
        for j in range(n):
            got = dsts[j].t.cpu().numpy()
            want = before[j].cpu().numpy()
            want[off:off + nbytes] = hosts[j][off:off + nbytes]
            assert np.array_equal(got, want), f"stream {j}"
            assert dsts[j].guards_intact()
