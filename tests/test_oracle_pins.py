"""Pins for the CPU oracle: each test checks the oracle against something
other than itself -- the pages' worked example, closed forms, torch's own
FP8/BF16 codecs, a brute-force nearest-value search, exact rational
arithmetic, and invariants of the encoding.

Sources: the RCCLX article (code-journey.com; pt and ko editions) --
"Core feature 1: Direct Data Access (DDA)" (DDA Flat, DDA Tree items),
"Core feature 2: Low-Precision Collectives" (opening paragraph: FP8, up to
4:1, messages >= 16MB; feature table rows "Data types" and "Compute
precision"), "Practical guide" (usage example).
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import rxgen as G

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

TORCH_FP8 = {O.E4M3: torch.float8_e4m3fn, O.E5M2: torch.float8_e5m2}
MAXCODE = {O.E4M3: 0x7E, O.E5M2: 0x7B}
FMAXV = {O.E4M3: 448.0, O.E5M2: 57344.0}


def f32(x):
    return np.asarray(x, dtype=np.float32)


def bits_to_f32(u):
    return np.asarray(u, dtype=np.uint32).view(np.float32)


def torch_decode_table(fmt):
    """Value of every code according to torch's float8 dtypes (independent
    of the oracle)."""
    codes = torch.arange(256, dtype=torch.uint8)
    return codes.view(TORCH_FP8[fmt]).float().numpy()


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------------------
# P1: the pages' worked example (rank-id fill, SUM) and its closed form
# ---------------------------------------------------------------------------

def test_p1_rank_id_example_golden():
    kv = {r[0]: r[1] for r in read_golden("rank_id_allreduce.txt")}
    n = int(kv["nsrc"])
    count = int(kv["rows"]) * int(kv["cols"])
    srcs = [G.fill(count, G.FP32, G.RANK, rank=r) for r in range(n)]
    y = O.reduce_flat(srcs, O.FP32)
    assert np.all(y == np.float32(float(kv["expected"])))


@pytest.mark.parametrize("dtype", [O.FP32, O.BF16])
@pytest.mark.parametrize("n", list(range(1, 17)))
def test_p1_rank_id_closed_form(n, dtype):
    srcs = [G.fill(200, dtype, G.RANK, rank=r) for r in range(n)]
    y = O.reduce_flat(srcs, dtype)
    if dtype == O.BF16:
        y = O.bf16_to_f32(y)
    assert np.all(y == n * (n - 1) // 2)


# ---------------------------------------------------------------------------
# P2: integer-valued inputs -> exact sums, any order
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 3, 8, 16])
def test_p2_integer_sum_fp32(n):
    count = 1000
    srcs = [G.fill(count, G.FP32, G.INT, seed=7, rank=r, param=1 << 20) for r in range(n)]
    exact = np.sum(np.stack([s.astype(np.int64) for s in srcs]), axis=0)
    y = O.reduce_flat(srcs, O.FP32)
    assert np.array_equal(y.astype(np.int64), exact)


@pytest.mark.parametrize("n", [1, 2, 5, 8])
def test_p2_integer_sum_bf16(n):
    count = 999
    srcs = [G.fill(count, G.BF16, G.INT, seed=8, rank=r, param=16) for r in range(n)]
    exact = np.sum(np.stack([O.bf16_to_f32(s).astype(np.int64) for s in srcs]), axis=0)
    y = O.bf16_to_f32(O.reduce_flat(srcs, O.BF16))
    # |sum| <= 128 is exactly representable in BF16 (8 significant bits)
    assert np.array_equal(y.astype(np.int64), exact)


# ---------------------------------------------------------------------------
# P3: FP32 accumulation and the fixed source order
# ---------------------------------------------------------------------------

def test_p3_fp32_accumulation_bf16():
    # BF16 sources {256, 1 x 7}: FP32 accumulation gives 263, which rounds
    # (tie, to even) to 264 in BF16; a BF16 accumulator would stay at 256.
    vals = [256.0] + [1.0] * 7
    srcs = [np.full(16, np.uint16(torch.tensor(v).bfloat16().view(torch.int16).item() & 0xFFFF))
            for v in vals]
    y = O.bf16_to_f32(O.reduce_flat(srcs, O.BF16))
    assert np.all(y == 264.0)
    assert torch.tensor(263.0).bfloat16().float().item() == 264.0
    bf_acc = torch.tensor(256.0).bfloat16()
    for _ in range(7):
        bf_acc = (bf_acc + torch.tensor(1.0).bfloat16()).bfloat16()
    assert bf_acc.float().item() == 256.0


def test_p3_left_fold_order_fp32():
    # ((1e8 + 1) - 1e8): 1e8 + 1 rounds back to 1e8 in FP32 (spacing 8), so
    # the left fold over (a, b, c) gives 0, while the fold over (a, c, b)
    # (b added last) gives 1: the result tells which order was folded.
    a = f32([1e8] * 4)
    b = f32([1.0] * 4)
    c = f32([-1e8] * 4)
    assert np.all(O.reduce_flat([a, b, c], O.FP32) == 0.0)
    assert np.all(O.reduce_flat([c, b, a], O.FP32) == 0.0)
    assert np.all(O.reduce_flat([a, c, b], O.FP32) == 1.0)
    assert np.all(O.reduce_flat([c, a, b], O.FP32) == 1.0)


def test_p3_negative_zero_start_value():
    # Starting from source 0 (not from +0): all -0 inputs stay -0.
    z = f32([-0.0] * 8)
    y = O.reduce_flat([z, z, z], O.FP32)
    assert np.all(np.signbit(y))


# ---------------------------------------------------------------------------
# P4: "up to 4:1" compression
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,block,ratio", [
    (O.FP32, 128, 32 / (8 + 32 / 128)),
    (O.FP32, 256, 32 / (8 + 32 / 256)),
    (O.BF16, 256, 16 / (8 + 32 / 256)),
])
def test_p4_compression_ratio(dtype, block, ratio):
    count = block * 64
    src = G.fill(count, dtype, G.NORMAL, seed=3)
    codes, scales = O.quant_fp8([src], dtype, O.E4M3, block)
    got = src.nbytes / (codes[0].nbytes + scales[0].nbytes)
    assert got == pytest.approx(ratio, rel=1e-12)
    assert got < 4.0
    if dtype == O.FP32:
        assert codes[0].nbytes * 4 == src.nbytes


# ---------------------------------------------------------------------------
# P5: all 256 codes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_p5_decode_matches_torch(fmt):
    mine = O.fp8_decode(np.arange(256, dtype=np.uint8), fmt)
    ref = torch_decode_table(fmt)
    nan_m, nan_r = np.isnan(mine), np.isnan(ref)
    assert np.array_equal(nan_m, nan_r)
    ok = ~nan_m
    assert np.array_equal(mine[ok].view(np.uint32), ref[ok].view(np.uint32))


def test_p5_landmarks():
    d4 = lambda c: float(O.fp8_decode(np.array([c], np.uint8), O.E4M3)[0])
    d5 = lambda c: float(O.fp8_decode(np.array([c], np.uint8), O.E5M2)[0])
    assert d4(0x7E) == 448.0 and d4(0x08) == 2.0 ** -6 and d4(0x01) == 2.0 ** -9
    assert math.isnan(d4(0x7F)) and math.isnan(d4(0xFF))
    assert d5(0x7B) == 57344.0 and d5(0x7C) == math.inf and d5(0x04) == 2.0 ** -14
    assert d5(0x01) == 2.0 ** -16
    assert all(math.isnan(d5(c)) for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF))
    assert O.fp8_max(O.E4M3) == 448.0 and O.fp8_max(O.E5M2) == 57344.0


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_p5_round_trip_every_code(fmt):
    codes = np.arange(256, dtype=np.uint8)
    vals = O.fp8_decode(codes, fmt)
    finite = np.isfinite(vals)
    back = O.fp8_encode(vals[finite], fmt)
    assert np.array_equal(back, codes[finite])
    assert O.fp8_encode(f32([-0.0]), fmt)[0] == 0x80
    if fmt == O.E5M2:
        assert list(O.fp8_encode(f32([np.inf, -np.inf]), fmt)) == [0x7B, 0xFB]


# ---------------------------------------------------------------------------
# P6: brute-force nearest representable value
# ---------------------------------------------------------------------------

def brute_force_encode(x, fmt):
    """Independent encode: nearest finite value of torch's decode table,
    ties to the even code, magnitudes at or beyond FMAX clamp to FMAX."""
    table = torch_decode_table(fmt).astype(np.float64)
    pos_codes = np.array([c for c in range(128) if np.isfinite(table[c])], np.int64)
    pos_vals = table[pos_codes]
    order = np.argsort(pos_vals, kind="stable")
    pos_codes, pos_vals = pos_codes[order], pos_vals[order]
    a = np.abs(x.astype(np.float64))
    a = np.minimum(a, pos_vals[-1])
    hi = np.searchsorted(pos_vals, a, side="left")
    hi = np.clip(hi, 0, len(pos_vals) - 1)
    lo = np.clip(hi - 1, 0, len(pos_vals) - 1)
    d_lo = a - pos_vals[lo]
    d_hi = pos_vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (pos_codes[hi] % 2 == 0))
    pick = np.where(pick_hi, hi, lo)
    exact = pos_vals[hi] == a
    pick = np.where(exact, hi, pick)
    code = pos_codes[pick].astype(np.uint8)
    sign = np.signbit(x).astype(np.uint8) << 7
    return code | sign


def _tie_neighbourhood(fmt, k=4):
    """FP32 values within k ulps of every midpoint between adjacent FP8
    values, and of every FP8 value."""
    table = torch_decode_table(fmt)
    vals = np.unique(table[np.isfinite(table)].astype(np.float32))
    vals = vals[vals >= 0]
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    pts = np.concatenate([vals, mids]).view(np.uint32).astype(np.int64)
    offs = np.arange(-k, k + 1)
    u = (pts[:, None] + offs[None, :]).ravel()
    u = u[(u >= 0) & (u < 0x7F800000)].astype(np.uint32)
    x = u.view(np.float32)
    return np.concatenate([x, -x])


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_p6_brute_force_ties_and_boundaries(fmt):
    x = _tie_neighbourhood(fmt)
    assert np.array_equal(O.fp8_encode(x, fmt), brute_force_encode(x, fmt))


@pytest.fixture(scope="module")
def fp8_sweep():
    """tests/bruteforce/fp8_sweep.c built for the host: an independent
    nearest-value search run over all 2^32 FP32 patterns on worker threads."""
    import ctypes
    import shutil
    import subprocess
    import tempfile
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    tmp = tempfile.mkdtemp()
    so = os.path.join(tmp, "libfp8sweep.so")
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "bruteforce", "fp8_sweep.c")
    r = subprocess.run([gcc, "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-pthread",
                        src, "-o", so, "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    L = ctypes.CDLL(so)
    U64 = ctypes.POINTER(ctypes.c_uint64)
    L.fp8_sweep.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, U64, U64,
                            ctypes.POINTER(ctypes.c_uint32)]
    L.fp8_sweep.restype = ctypes.c_int
    yield L
    shutil.rmtree(tmp, ignore_errors=True)


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_p6_brute_force_every_fp32_pattern(fmt, fp8_sweep):
    # Every FP32 bit pattern but the NaNs (4,278,190,082 values, both signs,
    # subnormals, +-0, +-Inf): the oracle's encoder against a nearest-value
    # search over torch's decode table, with ties to the even code and
    # saturation. About a minute per format on 8 host threads.
    import ctypes
    table = np.ascontiguousarray(torch_decode_table(fmt).astype(np.float32))
    encoder = ctypes.cast(O.lib().rxo_fp8_encode, ctypes.c_void_p)
    checked, bad, first = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint32()
    threads = max(1, min(os.cpu_count() or 1, 16))
    rc = fp8_sweep.fp8_sweep(table.ctypes.data, fmt, encoder, threads, ctypes.byref(checked),
                             ctypes.byref(bad), ctypes.byref(first))
    assert rc == 0
    assert checked.value == (1 << 32) - 2 * ((1 << 23) - 1)
    assert bad.value == 0, f"{bad.value} mismatches, first at FP32 bits {first.value:#010x}"


# ---------------------------------------------------------------------------
# P7: library cross-checks (torch CPU conversions; torch does not saturate,
# so compare on inputs clamped to [-FMAX, FMAX])
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_p7_torch_fp8_conversion(fmt):
    rng = np.random.default_rng(11)
    n = 2_000_000
    mags = rng.uniform(-20, 17, size=n)
    x = (np.exp2(mags) * rng.choice([-1.0, 1.0], size=n)).astype(np.float32)
    x = np.clip(x, -FMAXV[fmt], FMAXV[fmt])
    ref = torch.from_numpy(x).to(TORCH_FP8[fmt]).view(torch.uint8).numpy()
    assert np.array_equal(O.fp8_encode(x, fmt), ref)


def test_p7_torch_bf16_conversion():
    rng = np.random.default_rng(12)
    u = rng.integers(0, 0x7F800000, size=4_000_000, dtype=np.uint32)
    # add exact ties and their neighbours
    ties = (rng.integers(0, 0x7F7F, size=100_000, dtype=np.uint32) << 16) | 0x8000
    u = np.concatenate([u, ties, ties + 1, ties - 1])
    x = u.view(np.float32)
    x = np.concatenate([x, -x])
    ref = torch.from_numpy(x).bfloat16().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16(x), ref)


def test_p7_torch_bf16_conversion_every_pattern():
    # Every FP32 bit pattern but the NaNs, in chunks of 2^26: the oracle's
    # round-to-nearest-even narrowing against torch's (values near the top
    # of the range round to +-Inf in both). About half a minute.
    step = 1 << 26
    for start in range(0, 1 << 32, step):
        u = np.arange(start, start + step, dtype=np.uint64).astype(np.uint32)
        x = u.view(np.float32)
        ref = torch.from_numpy(x).bfloat16().view(torch.int16).numpy().view(np.uint16)
        got = O.f32_to_bf16(x)
        if (start & 0x7FFFFFFF) + step > 0x7F800000:    # the chunk holds NaN patterns
            keep = ~np.isnan(x)
            got, ref = got[keep], ref[keep]
        assert np.array_equal(got, ref), f"chunk at {start:#010x}"


def test_p7_bf16_widening_exact():
    h = np.arange(0, 0x7F80, dtype=np.uint16)
    ref = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(O.bf16_to_f32(h).view(np.uint32), ref.view(np.uint32))


# ---------------------------------------------------------------------------
# Block scale: correctly rounded divisions, checked with exact rationals
# ---------------------------------------------------------------------------

def _is_correctly_rounded_f32(q: float, exact: Fraction) -> bool:
    qf = np.float32(q)
    below = np.nextafter(qf, np.float32(-np.inf))
    above = np.nextafter(qf, np.float32(np.inf))
    err = abs(Fraction(float(qf)) - exact)
    return (err <= abs(Fraction(float(below)) - exact)
            and err <= abs(Fraction(float(above)) - exact))


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_block_scale_exact_rationals(fmt):
    rng = np.random.default_rng(5)
    fm = Fraction(FMAXV[fmt])
    for _ in range(400):
        x = (rng.standard_normal(rng.integers(1, 300)) *
             np.exp2(rng.uniform(-30, 30))).astype(np.float32)
        s, r = O.block_scale(x, fmt)
        a = Fraction(float(np.max(np.abs(x))))
        assert a == max(Fraction(float(v)) for v in np.abs(x))
        assert _is_correctly_rounded_f32(s, a / fm)
        assert _is_correctly_rounded_f32(r, fm / a)


@pytest.fixture(scope="module")
def scale_sweep():
    """tests/bruteforce/scale_sweep.c built for the host: exact checks of
    correctly rounded division over every non-negative finite FP32 A."""
    import ctypes
    import shutil
    import subprocess
    import tempfile
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    tmp = tempfile.mkdtemp()
    so = os.path.join(tmp, "libscalesweep.so")
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "bruteforce", "scale_sweep.c")
    r = subprocess.run([gcc, "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-pthread",
                        src, "-o", so, "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    L = ctypes.CDLL(so)
    U64 = ctypes.POINTER(ctypes.c_uint64)
    L.scale_sweep.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_void_p, ctypes.c_int, U64, U64,
                              ctypes.POINTER(ctypes.c_uint32)]
    L.scale_sweep.restype = ctypes.c_int
    yield L
    shutil.rmtree(tmp, ignore_errors=True)


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_block_scale_every_absmax(fmt, scale_sweep):
    # Every non-negative finite FP32 block absmax A (2,139,095,040 values):
    # s and r correctly rounded (ties to even), checked with exact products,
    # and s = r = 1 exactly on the degenerate blocks. ~20 s per format.
    import ctypes
    entry = ctypes.cast(O.lib().rxo_block_scale_bits_range, ctypes.c_void_p)
    checked, bad, first = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint32()
    threads = max(1, min(os.cpu_count() or 1, 16))
    rc = scale_sweep.scale_sweep(fmt, FMAXV[fmt], entry, threads, ctypes.byref(checked),
                                 ctypes.byref(bad), ctypes.byref(first))
    assert rc == 0
    assert checked.value == 0x7F7FFFFF + 1
    assert bad.value == 0, f"{bad.value} wrong scales, first at A bits {first.value:#010x}"


@pytest.fixture(scope="module")
def kernel_scale_sweep():
    """tests/bruteforce/block_scale_sweep.c built for the host: the kernels'
    division-free block scale repeated in host FP32 against IEEE division."""
    import ctypes
    import shutil
    import subprocess
    import tempfile
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    tmp = tempfile.mkdtemp()
    so = os.path.join(tmp, "libkscalesweep.so")
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "bruteforce", "block_scale_sweep.c")
    r = subprocess.run([gcc, "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
                        "-pthread", src, "-o", so, "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    L = ctypes.CDLL(so)
    U64 = ctypes.POINTER(ctypes.c_uint64)
    L.block_scale_sweep.argtypes = [ctypes.c_float, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                    ctypes.c_int, U64, U64, ctypes.POINTER(ctypes.c_uint32)]
    L.block_scale_sweep.restype = ctypes.c_int
    yield L
    shutil.rmtree(tmp, ignore_errors=True)


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_kernel_block_scale_arithmetic(fmt, kernel_scale_sweep):
    # The FMA-corrected quotients the kernels use for s and r, with every
    # reciprocal estimate within 1 ulp: every 61st A pattern up to +inf, and
    # every pattern in the ranges where the steps could break down (tiny A,
    # where s is subnormal and r overflows; A within four binades of
    # FLT_MAX, where 1 / A is subnormal). The full sweep of all 2^31 patterns
    # (step 1 over [0, 0x7F800001)) also finds no mismatch; it takes about
    # 1.5 minutes on 8 threads.
    import ctypes
    threads = max(1, min(os.cpu_count() or 1, 16))
    for lo, hi, step in ((0, 0x7F800001, 61), (0, 0x01000000, 1), (0x7D800000, 0x7F800001, 1)):
        checked, bad, first = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint32()
        rc = kernel_scale_sweep.block_scale_sweep(FMAXV[fmt], lo, hi, step, threads, ctypes.byref(checked),
                                                  ctypes.byref(bad), ctypes.byref(first))
        assert rc == 0 and checked.value == 3 * (-(-(hi - lo) // step))
        assert bad.value == 0, f"[{lo:#x}, {hi:#x}) step {step}: {bad.value} mismatches, first A bits {first.value:#010x}"


def test_block_scale_degenerate():
    for fmt in (O.E4M3, O.E5M2):
        assert O.block_scale(f32([0.0, -0.0, 0.0]), fmt) == (1.0, 1.0)
        # A so small that FMAX / A overflows FP32
        assert O.block_scale(f32([1e-40, -2e-40]), fmt) == (1.0, 1.0)
        s, r = O.block_scale(f32([1.0]), fmt)
        assert s > 0 and r == FMAXV[fmt]


# ---------------------------------------------------------------------------
# Quantizer: each code is the brute-force nearest value of fl32(x * r)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,fmt,block", [
    (O.FP32, O.E4M3, 128), (O.BF16, O.E5M2, 256), (O.FP32, O.E5M2, 32),
    (O.BF16, O.E4M3, 64)])
def test_quant_codes_brute_force(dtype, fmt, block):
    count = block * 37 + 5  # ragged last block
    src = G.fill(count, dtype, G.NORMAL_OUTLIER, seed=21)
    x = src if dtype == O.FP32 else O.bf16_to_f32(src)
    codes, scales = O.quant_fp8([src], dtype, fmt, block)
    nb = (count + block - 1) // block
    assert scales[0].size == nb
    for b in range(nb):
        xb = x[b * block:(b + 1) * block]
        a = np.float32(np.max(np.abs(xb)))
        r = np.float32(FMAXV[fmt]) / a  # one IEEE division, same as the oracle's reading
        y = (xb * r).astype(np.float32)
        assert np.array_equal(codes[0][b * block:(b + 1) * block], brute_force_encode(y, fmt))
        assert scales[0][b] == np.float32(a / np.float32(FMAXV[fmt]))


# ---------------------------------------------------------------------------
# P8: composition identities
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt,block", [(O.E4M3, 128), (O.E5M2, 256), (O.E4M3, 32)])
def test_p8_drr_sum_is_flat_of_dequant(fmt, block):
    n, count = 5, block * 9 + 3
    srcs = [G.fill(count, G.FP32, G.NORMAL, seed=31, rank=r) for r in range(n)]
    codes, scales = O.quant_fp8(srcs, O.FP32, fmt, block)
    _, _, s_hp = O.dequant_reduce_requant(codes, scales, fmt, block, O.DRR_SUM, O.FP32)
    deq = []
    for c, s in zip(codes, scales):
        d = O.fp8_decode(c, fmt)
        deq.append((d * np.repeat(s, block)[:count]).astype(np.float32))
    assert np.array_equal(s_hp.view(np.uint32), O.reduce_flat(deq, O.FP32).view(np.uint32))
    # REQUANT == quant(SUM); its hp output == dequant of the requantized codes
    oc, osc, ohp = O.dequant_reduce_requant(codes, scales, fmt, block, O.DRR_REQUANT, O.FP32)
    qc, qs = O.quant_fp8([s_hp], O.FP32, fmt, block)
    assert np.array_equal(oc, qc[0]) and np.array_equal(osc, qs[0])
    d2 = (O.fp8_decode(oc, fmt) * np.repeat(osc, block)[:count]).astype(np.float32)
    assert np.array_equal(ohp.view(np.uint32), d2.view(np.uint32))
    _, _, ohp16 = O.dequant_reduce_requant(codes, scales, fmt, block, O.DRR_REQUANT, O.BF16)
    assert np.array_equal(ohp16, O.f32_to_bf16(d2))


def test_p8_tree_partition_brute_force():
    for dtype, vec in ((O.FP32, 4), (O.BF16, 8)):
        for n in range(1, 17):
            for count in range(0, 65):
                covered = np.zeros(count, dtype=np.int64)
                bounds = [O.tree_chunk(count, n, dtype, k) for k in range(n)]
                for lo, hi in bounds:
                    assert 0 <= lo <= hi <= count
                    # every chunk starts on a 16-byte boundary
                    assert lo % vec == 0 or lo == count
                    covered[lo:hi] += 1
                # disjoint cover of [0, count), chunks in rank order
                assert np.all(covered == 1)
                assert all(bounds[k][1] <= bounds[k + 1][0] or bounds[k + 1][0] == bounds[k + 1][1]
                           for k in range(n - 1))
                if not count:
                    continue
                lens = [hi - lo for lo, hi in bounds]
                c = max(lens)
                last = max(k for k in range(n) if lens[k])
                # all chunks before the last non-empty one are full-length
                assert all(lens[k] == c for k in range(last))
                # balance: the smallest vec-multiple length that covers count
                cc = -(-c // vec) * vec
                assert cc * n >= count and (cc - vec) * n < count


@pytest.mark.parametrize("dtype", [O.FP32, O.BF16])
def test_p8_tree_chunks_union_equals_flat(dtype):
    n, count = 6, 1237
    srcs = [G.fill(count, dtype, G.NORMAL, seed=41, rank=r) for r in range(n)]
    flat = O.reduce_flat(srcs, dtype)
    sentinel = 0x7FC1 if dtype == O.BF16 else np.float32(12345.5)
    npdt = np.uint16 if dtype == O.BF16 else np.float32
    union = np.full(count, sentinel, dtype=npdt)
    for k in range(n):
        dsts = [np.full(count, sentinel, dtype=npdt) for _ in range(n)]
        O.reduce_scatter_chunk_bcast(srcs, dtype, k, dsts)
        lo, hi = O.tree_chunk(count, n, dtype, k)
        for d in dsts:
            assert np.array_equal(d[lo:hi], flat[lo:hi])
            assert np.all(d[:lo] == sentinel) and np.all(d[hi:] == sentinel)
        union[lo:hi] = dsts[0][lo:hi]
    assert np.array_equal(union, flat)


def test_p8_single_source_is_copy():
    for dtype in (O.FP32, O.BF16):
        x = G.fill(333, dtype, G.NORMAL, seed=51)
        assert np.array_equal(O.reduce_flat([x], dtype), x)


# ---------------------------------------------------------------------------
# P9: code invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,fmt,block", [(O.FP32, O.E4M3, 128), (O.BF16, O.E5M2, 256)])
def test_p9_code_invariants(dtype, fmt, block):
    count = block * 50
    srcs = [G.fill(count, dtype, G.LAPLACE, seed=61, rank=r) for r in range(3)]
    codes, scales = O.quant_fp8(srcs, dtype, fmt, block)
    dec = torch_decode_table(fmt)
    for c, s in zip(codes, scales):
        assert not np.any(np.isnan(dec[c]))
        assert np.all(s > 0)
        per_block = (c & 0x7F).reshape(-1, block)
        assert np.all(np.any(per_block == MAXCODE[fmt], axis=1))


# ---------------------------------------------------------------------------
# P10: the worked example through the low-precision path (golden)
# ---------------------------------------------------------------------------

def test_p10_rank_id_lowprec_golden():
    n, count = 8, 200
    for fmt_s, block_s, maxc_s, s2_s, res_s in read_golden("rank_id_lowprec.txt"):
        fmt, block, maxc = O.FMT[fmt_s], int(block_s), int(maxc_s, 16)
        srcs = [G.fill(count, G.FP32, G.RANK, rank=r) for r in range(n)]
        codes, scales = O.quant_fp8(srcs, O.FP32, fmt, block)
        assert np.all(codes[0] == 0x00) and np.all(scales[0] == 1.0)
        for r in range(1, n):
            assert np.all(codes[r] == maxc)
        oc, osc, ohp = O.dequant_reduce_requant(codes, scales, fmt, block,
                                                O.DRR_REQUANT, O.FP32)
        assert np.all(osc == np.float32(float(s2_s)))
        assert np.all(oc == maxc)
        assert np.all(ohp == np.float32(float(res_s)))


# ---------------------------------------------------------------------------
# P11: error bounds of the low-precision path against the unquantized sum
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("wl,fmt,block,u,uprime", [
    ("lp_fp32", O.E4M3, 128, 2.0 ** -4, 1 / 28),
    ("lp_bf16", O.E5M2, 256, 2.0 ** -3, 1 / 14),
])
def test_p11_error_bounds(wl, fmt, block, u, uprime):
    w = G.WORKLOADS[wl]
    count = block * 512
    srcs = [w.source(r, count=count) for r in range(w.nsrc)]
    n = w.nsrc
    x = [s if w.dtype == O.FP32 else O.bf16_to_f32(s) for s in srcs]
    T = O.reduce_flat([xi.astype(np.float32) for xi in x], O.FP32).astype(np.float64)
    codes, scales = O.quant_fp8(srcs, w.dtype, fmt, block)
    _, _, S = O.dequant_reduce_requant(codes, scales, fmt, block, O.DRR_SUM, O.FP32)
    _, _, D = O.dequant_reduce_requant(codes, scales, fmt, block, O.DRR_REQUANT, O.FP32)
    X = np.stack([xi.astype(np.float64) for xi in x])            # (n, count)
    Ab_r = np.abs(X).reshape(n, -1, block).max(axis=2)           # (n, nb)
    Ab = np.repeat(Ab_r.max(axis=0), block)                      # per element
    S64, D64 = S.astype(np.float64), D.astype(np.float64)
    # B1: |S - T| <= N u A_b
    assert np.all(np.abs(S64 - T) <= n * u * Ab)
    # B2: per-term bound of quantization, requantization and FP32 roundings
    Abr = np.repeat(Ab_r, block, axis=1)
    A2 = np.repeat(np.abs(S64).reshape(-1, block).max(axis=1), block)
    b2 = (np.minimum(u * np.abs(X), Abr * uprime).sum(axis=0)
          + np.minimum(u * np.abs(S64), A2 * uprime)
          + n * 2.0 ** -22 * np.abs(X).sum(axis=0))
    assert np.all(np.abs(D64 - T) <= b2)
    # the literal per-element bound N * u * blockabsmax, on these inputs
    assert np.all(np.abs(D64 - T) <= n * u * Ab)


# ---------------------------------------------------------------------------
# Low-precision tree step: chunks are whole blocks; the chunks of all ranks
# together reproduce the requantized allreduce; nothing outside the chunk
# is written
# ---------------------------------------------------------------------------

def test_lp_tree_partition_brute_force():
    for block in (32, 128, 1024):
        for n in range(1, 17):
            for count in list(range(0, 70)) + [block * 5 + 3, block * 16, block * 33 + 1]:
                bounds = [O.lp_tree_chunk(count, n, block, k) for k in range(n)]
                covered = np.zeros(count, dtype=np.int64)
                for lo, hi in bounds:
                    assert 0 <= lo <= hi <= count
                    assert lo % block == 0 or lo == count
                    covered[lo:hi] += 1
                assert np.all(covered == 1)
                if count:
                    lens = [hi - lo for lo, hi in bounds]
                    c = max(lens)
                    last = max(k for k in range(n) if lens[k])
                    assert all(lens[k] == c for k in range(last))
                    cc = -(-c // block) * block
                    assert cc * n >= count and (cc - block) * n < count


@pytest.mark.parametrize("fmt,block", [(O.E4M3, 128), (O.E5M2, 256), (O.E4M3, 32)])
def test_lp_tree_union_is_requantized_allreduce(fmt, block):
    n, count = 5, block * 23 + 9
    srcs = [G.fill(count, G.FP32, G.NORMAL_OUTLIER, seed=71, rank=r) for r in range(n)]
    codes, scales = O.quant_fp8(srcs, O.FP32, fmt, block)
    ref_c, ref_s, ref_h = O.dequant_reduce_requant(codes, scales, fmt, block, O.DRR_REQUANT,
                                                   O.BF16, True)
    nb = -(-count // block)
    union_c = np.full(count, 0xA5, np.uint8)
    union_s = np.full(nb, -7.0, np.float32)
    union_h = np.full(count, 0x7FA5, np.uint16)
    for k in range(n):
        dc = [np.full(count, 0xA5, np.uint8) for _ in range(n)]
        ds = [np.full(nb, -7.0, np.float32) for _ in range(n)]
        hp = np.full(count, 0x7FA5, np.uint16)
        O.lp_reduce_scatter_chunk_bcast(codes, scales, fmt, block, k, dc, ds, hp, O.BF16)
        lo, hi = O.lp_tree_chunk(count, n, block, k)
        b0, b1 = lo // block, -(-hi // block)
        for j in range(n):
            assert np.array_equal(dc[j][lo:hi], ref_c[lo:hi])
            assert np.all(dc[j][:lo] == 0xA5) and np.all(dc[j][hi:] == 0xA5)
            assert np.array_equal(ds[j][b0:b1], ref_s[b0:b1])
            assert np.all(ds[j][:b0] == -7.0) and np.all(ds[j][b1:] == -7.0)
        assert np.array_equal(hp[lo:hi], ref_h[lo:hi])
        assert np.all(hp[:lo] == 0x7FA5) and np.all(hp[hi:] == 0x7FA5)
        union_c[lo:hi] = dc[0][lo:hi]
        union_s[b0:b1] = ds[0][b0:b1]
        union_h[lo:hi] = hp[lo:hi]
    assert np.array_equal(union_c, ref_c) and np.array_equal(union_s, ref_s)
    assert np.array_equal(union_h, ref_h)


def test_lp_tree_rank_id_example():
    # the pages' rank-id example through the low-precision tree: every chunk
    # requantizes to the max code with scale 28/FMAX and dequantizes to 28
    n, count = 8, 200
    for fmt_s, block_s, maxc_s, s2_s, res_s in read_golden("rank_id_lowprec.txt"):
        fmt, block, maxc = O.FMT[fmt_s], int(block_s), int(maxc_s, 16)
        srcs = [G.fill(count, G.FP32, G.RANK, rank=r) for r in range(n)]
        codes, scales = O.quant_fp8(srcs, O.FP32, fmt, block)
        nb = -(-count // block)
        dc = [np.zeros(count, np.uint8) for _ in range(n)]
        ds = [np.zeros(nb, np.float32) for _ in range(n)]
        hp = np.zeros(count, np.float32)
        for k in range(n):
            O.lp_reduce_scatter_chunk_bcast(codes, scales, fmt, block, k, dc, ds, hp, O.FP32)
        for j in range(n):
            assert np.all(dc[j] == maxc) and np.all(ds[j] == np.float32(float(s2_s)))
        assert np.all(hp == np.float32(float(res_s)))


# ---------------------------------------------------------------------------
# Local allreduce (all ranks' buffers on one device), in place
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("algo", [O.ALGO_FLAT, O.ALGO_TREE, O.ALGO_LOWPREC])
def test_allreduce_local_rank_id_example(algo):
    # the pages' usage example: 8 ranks, 10x20 FP32 filled with the rank id,
    # SUM in place -> 28 in every rank's tensor, whatever the algorithm
    for fmt, block in ((O.E4M3, 128), (O.E5M2, 256)):
        bufs = [G.fill(200, G.FP32, G.RANK, rank=r) for r in range(8)]
        O.allreduce_local(bufs, O.FP32, algo, fmt, block)
        for b in bufs:
            assert np.all(b == 28.0)


@pytest.mark.parametrize("dtype", [O.FP32, O.BF16])
def test_allreduce_local_flat_and_tree_broadcast_the_reduce(dtype):
    n, count = 6, 3001
    srcs = [G.fill(count, dtype, G.NORMAL, seed=81, rank=r) for r in range(n)]
    ref = O.reduce_flat(srcs, dtype)
    for algo in (O.ALGO_FLAT, O.ALGO_TREE):
        bufs = [s.copy() for s in srcs]
        O.allreduce_local(bufs, dtype, algo)
        for b in bufs:
            assert np.array_equal(b, ref)


@pytest.mark.parametrize("dtype,fmt,block", [(O.FP32, O.E4M3, 128), (O.BF16, O.E5M2, 256)])
def test_allreduce_local_lowprec_is_requantized_allreduce(dtype, fmt, block):
    # every rank ends with dequant(requant(sum)): the high-precision output of
    # the dequant-reduce-requant step on the quantized inputs
    n, count = 5, block * 13 + 7
    srcs = [G.fill(count, dtype, G.LAPLACE, seed=82, rank=r) for r in range(n)]
    codes, scales = O.quant_fp8(srcs, dtype, fmt, block)
    _, _, ref = O.dequant_reduce_requant(codes, scales, fmt, block, O.DRR_REQUANT, dtype, True)
    bufs = [s.copy() for s in srcs]
    O.allreduce_local(bufs, dtype, O.ALGO_LOWPREC, fmt, block)
    for b in bufs:
        assert np.array_equal(b, ref)
