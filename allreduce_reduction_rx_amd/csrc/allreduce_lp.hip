// allreduce_lp.hip -- the one-device low-precision allreduce in one pass
// (RCCLX article, code-journey.com, "Core feature 2: Low-Precision
// Collectives": FP8 quantization of FP32/BF16, FP32 compute; "Practical
// guide": allreduce SUM in place).
//
// On one device every rank's quantization, the reduce-scatter of the FP8
// chunks, their requantization and every rank's dequantization of the
// gathered message are block-local, so one wave does all of it for a tile of
// every rank's buffer in registers: load the N ranks' 16-byte vectors,
// quantize each rank's block exactly as the quantizer does (block absmax
// across the lanes of the block, s = A / FMAX, r = FMAX / A, saturating RNE
// conversion), dequantize (decode x s, multiply and add kept separate), sum
// in rank order in FP32, requantize the sum, dequantize it and store the
// result into all N buffers. The codes never reach memory: N reads and N
// writes of the message per element, against 2N plus the codes' round trip
// for a quantize pass followed by a reduce pass.
#include <array>
#include <utility>

#include "rx_device.hpp"
#include "rx_internal.hpp"

namespace rx {
namespace {

// A lane's share of one buffer: LB = 16 or 8 bytes.
template <int LB>
struct LaneVec;
template <>
struct LaneVec<16> {
    using T = u32x4;
};
template <>
struct LaneVec<8> {
    using T = u32x2;
};

// Widen a lane's LB bytes to VE floats (exact).
template <int DT, int W, typename V>
__device__ __forceinline__ void widen_lane(const V& x, float* f)
{
#pragma unroll
    for (int k = 0; k < W; ++k) {
        if constexpr (DT == 0) {
            f[k] = bits_f32(x[k]);
        } else {
            f[2 * k] = bf16_lo(x[k]);
            f[2 * k + 1] = bf16_hi(x[k]);
        }
    }
}

// Elements [e, count) of a partial lane vector, the rest zero (neutral for
// the block absmax; never stored). Every element is loaded from an index
// clamped to count - 1 (in bounds, count >= 1) and masked afterwards, so the
// loads carry no branches and are all in flight before the first use.
template <int DT, int W, typename V>
__device__ __forceinline__ V load_tail(const void* src, size_t e, size_t count)
{
    V x = {};
    if constexpr (DT == 0) {
        const uint32_t* p = static_cast<const uint32_t*>(src);
        uint32_t w[W];
#pragma unroll
        for (int k = 0; k < W; ++k)
            w[k] = p[e + k < count ? e + k : count - 1];
#pragma unroll
        for (int k = 0; k < W; ++k)
            x[k] = e + k < count ? w[k] : 0u;
    } else {
        const uint16_t* p = static_cast<const uint16_t*>(src);
        uint32_t h[2 * W];
#pragma unroll
        for (int k = 0; k < 2 * W; ++k)
            h[k] = p[e + k < count ? e + k : count - 1];
#pragma unroll
        for (int k = 0; k < 2 * W; ++k)
            x[k / 2] |= (e + k < count ? h[k] : 0u) << (16 * (k & 1));
    }
    return x;
}

// dequant(quant(f)) of the VE values of one lane, for a block whose absmax
// over its LPB lanes is taken here: out[k] = fl32(decode(code_k) * s). The
// codes are converted and decoded two at a time (both conversions work
// element by element, so the pairing does not change any result).
template <int F, int LPB, int VE>
__device__ __forceinline__ void quant_dequant(const float* f, float* out)
{
    float m = __builtin_fabsf(f[0]);
#pragma unroll
    for (int k = 1; k < VE; ++k)
        m = __builtin_fmaxf(m, __builtin_fabsf(f[k]));
    const float A = bits_f32(group_max<LPB>(__builtin_bit_cast(uint32_t, m)));
    float s, r;
    block_scale<F>(A, s, r);
#pragma unroll
    for (int q = 0; q < VE / 2; ++q) {
        const float y0 = clamp_fmax<F>(f[2 * q] * r);
        const float y1 = clamp_fmax<F>(f[2 * q + 1] * r);
        f32x2 d;
        if constexpr (F == kE4M3)
            d = __builtin_amdgcn_cvt_pk_f32_fp8(__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false), false);
        else
            d = __builtin_amdgcn_cvt_pk_f32_bf8(__builtin_amdgcn_cvt_pk_bf8_f32(y0, y1, 0, false), false);
        out[2 * q] = d[0] * s;
        out[2 * q + 1] = d[1] * s;
    }
}

// One wave per tile of 64 lane vectors of every rank (lane l: lane vector
// tile * 64 + l of LB bytes); a block spans LPB = BLOCK / VE <= 64 lanes of
// one tile.
// ONE: the message is whole tiles and the grid has a wave for each (decode
// size): one tile per wave, no loop and no partial-tile path (8 x 256K BF16
// E5M2/256 with 8-byte lanes: 4.06 -> 3.88 us).
template <int DT, int F, int BLOCK, int N, int LB, bool ONE = false>
__global__ __launch_bounds__(256) void k_allreduce_lp(AllreduceLpArgs a)
{
    using V = typename LaneVec<LB>::T;
    constexpr int W = LB / 4;                      // 32-bit words per lane vector
    constexpr int VE = DT == 0 ? W : 2 * W;        // elements per lane vector
    constexpr int LPB = BLOCK / VE;
    static_assert(LPB >= 1 && LPB <= kWave, "a block lies in the lanes of one wave");
    constexpr size_t kTileElems = (size_t)kWave * VE;
    const int lane = lane_id();
    const uint32_t wave_in_wg = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t waves_per_wg = blockDim.x / kWave;
    const uint32_t wg = a.xcd_ranges ? xcd_contiguous(blockIdx.x, gridDim.x) : blockIdx.x;
    const size_t wave = (size_t)wg * waves_per_wg + wave_in_wg;
    const size_t nwaves = (size_t)gridDim.x * waves_per_wg;
    const size_t ntiles = ONE ? a.count / kTileElems : (a.count + kTileElems - 1) / kTileElems;

    for (size_t t = wave; t < ntiles; t += nwaves) {
        const size_t v = t * kWave + lane;
        const size_t e = v * VE;
        const bool full = ONE || (t + 1) * kTileElems <= a.count;   // uniform
        V x[N];
        if (full) {
#pragma unroll
            for (int r = 0; r < N; ++r)
                x[r] = __builtin_nontemporal_load(static_cast<const V*>(a.buf[r]) + v);
        } else {
            // the one partial tile: element loads of every rank, no branches
#pragma unroll
            for (int r = 0; r < N; ++r)
                x[r] = load_tail<DT, W, V>(a.buf[r], e, a.count);
        }

        // every rank's block quantized and dequantized, folded in rank order
        float S[VE];
        {
            float f[VE];
            widen_lane<DT, W>(x[0], f);
            quant_dequant<F, LPB, VE>(f, S);
        }
#pragma unroll
        for (int r = 1; r < N; ++r) {
            float f[VE], d[VE];
            widen_lane<DT, W>(x[r], f);
            quant_dequant<F, LPB, VE>(f, d);
#pragma unroll
            for (int k = 0; k < VE; ++k)
                S[k] = S[k] + d[k];
        }
        // the requantized sum, dequantized: every rank's result
        float h[VE];
        quant_dequant<F, LPB, VE>(S, h);
        V y;
#pragma unroll
        for (int k = 0; k < W; ++k) {
            if constexpr (DT == 0)
                y[k] = __builtin_bit_cast(uint32_t, h[k]);
            else
                y[k] = pack_bf16(h[2 * k], h[2 * k + 1]);
        }
        if (full) {
#pragma unroll
            for (int r = 0; r < N; ++r)
                __builtin_nontemporal_store(y, static_cast<V*>(a.buf[r]) + v);
        } else if (e + VE <= a.count) {
#pragma unroll
            for (int r = 0; r < N; ++r)
                static_cast<V*>(a.buf[r])[v] = y;
        } else {
#pragma unroll
            for (int r = 0; r < N; ++r) {
#pragma unroll
                for (int k = 0; k < VE; ++k) {
                    if (e + k < a.count) {
                        if constexpr (DT == 0)
                            static_cast<uint32_t*>(a.buf[r])[e + k] = y[k];
                        else
                            static_cast<uint16_t*>(a.buf[r])[e + k] =
                                (uint16_t)(y[k / 2] >> (16 * (k & 1)));
                    }
                }
            }
        }
        if constexpr (ONE)
            break;
    }
}

using LpFn = void (*)(AllreduceLpArgs);

template <int DT, int F, int BLOCK, int LB, int... I>
constexpr std::array<LpFn, sizeof...(I)> lp_row(std::integer_sequence<int, I...>)
{
    return {{&k_allreduce_lp<DT, F, BLOCK, I + 1, LB>...}};
}
template <int DT, int F, int BLOCK, int LB, int... I>
constexpr std::array<LpFn, sizeof...(I)> lp_one_row(std::integer_sequence<int, I...>)
{
    return {{&k_allreduce_lp<DT, F, BLOCK, I + 1, LB, true>...}};
}

// Rows by block size (32, 64, ...): blocks of at most 64 lane vectors, with
// 16-byte lanes FP32 32..256 and BF16 32..512 (larger blocks use the
// two-pass path).
template <int DT, int F>
struct LpTable {
    static constexpr int kRows = DT == 0 ? 4 : 5;
    std::array<LpFn, kMaxSrc> row[kRows];
};

template <int DT, int F>
LpTable<DT, F> make_lp_table()
{
    const auto seq = std::make_integer_sequence<int, kMaxSrc>{};
    LpTable<DT, F> t{};
    t.row[0] = lp_row<DT, F, 32, 16>(seq);
    t.row[1] = lp_row<DT, F, 64, 16>(seq);
    t.row[2] = lp_row<DT, F, 128, 16>(seq);
    t.row[3] = lp_row<DT, F, 256, 16>(seq);
    if constexpr (DT == 1)
        t.row[4] = lp_row<DT, F, 512, 16>(seq);
    return t;
}

const LpTable<0, 0> kLpF32E4 = make_lp_table<0, 0>();
const LpTable<0, 1> kLpF32E5 = make_lp_table<0, 1>();
const LpTable<1, 0> kLpB16E4 = make_lp_table<1, 0>();
const LpTable<1, 1> kLpB16E5 = make_lp_table<1, 1>();

// 8-byte lanes (4 BF16 elements), for decode-size BF16 messages: twice the
// waves, each with half the per-element work. Blocks 32..256.
template <int F>
struct LpNarrowTable {
    std::array<LpFn, kMaxSrc> row[4];
    std::array<LpFn, kMaxSrc> one[4];   // messages of whole tiles, one tile per wave
};

template <int F>
LpNarrowTable<F> make_lp_narrow_table()
{
    const auto seq = std::make_integer_sequence<int, kMaxSrc>{};
    LpNarrowTable<F> t{};
    t.row[0] = lp_row<1, F, 32, 8>(seq);
    t.row[1] = lp_row<1, F, 64, 8>(seq);
    t.row[2] = lp_row<1, F, 128, 8>(seq);
    t.row[3] = lp_row<1, F, 256, 8>(seq);
    t.one[0] = lp_one_row<1, F, 32, 8>(seq);
    t.one[1] = lp_one_row<1, F, 64, 8>(seq);
    t.one[2] = lp_one_row<1, F, 128, 8>(seq);
    t.one[3] = lp_one_row<1, F, 256, 8>(seq);
    return t;
}

const LpNarrowTable<0> kLpB16E4Narrow = make_lp_narrow_table<0>();
const LpNarrowTable<1> kLpB16E5Narrow = make_lp_narrow_table<1>();

// Launch shape by the number of 16-byte-lane tiles T (measured on MI355X,
// 8 ranks, HBM-cold rotating buffers):
//  - T <= 8 per CU, BF16, blocks <= 256: 8-byte lanes, one tile per wave in
//    256-thread workgroups, each XCD a contiguous range (8 x 512 KiB
//    E5M2/256: 4.2 us against 4.8 us with 16-byte lanes; 8 x 1 MiB 5.09 ->
//    4.89 us, 8 x 2 MiB 7.26 -> 7.16 against 16-byte lanes below; at 16 per
//    CU 16-byte lanes were faster, 14.6 against 15.2 us at 8 x 4 MiB);
//  - T <= 16 per CU: 256-thread workgroups, at most 2 per CU (8 x 2 MiB FP32
//    E4M3/128: 6.9 us against 9.5 us; 8 x 4 MiB BF16: 14.8 against 15.3);
//  - larger: four 64-thread workgroups per CU (one wave per SIMD),
//    grid-stride: 8 x 512 MiB BF16 E5M2/256 1480 us (two 256-thread
//    workgroups per CU: 1942 us; five or three 64-thread ones: 1691,
//    1879 us), 8 x 64 MiB FP32 E4M3/128 180 us (207 us).
LaunchPolicy policy_lp_narrow() { return {256u, 256u, 0u}; }
LaunchPolicy policy_lp_medium() { return {256u, 256u, 2u}; }
LaunchPolicy policy_lp_large() { return {64u, 64u, 4u}; }

}  // namespace

bool allreduce_lp_fits(int dtype, int block)
{
    return block <= (dtype == 0 ? 256 : 512);
}

hipError_t launch_allreduce_lp(const AllreduceLpArgs& a, int nsrc, int dtype, int fmt, int block,
                               hipStream_t s)
{
    if (!allreduce_lp_fits(dtype, block))
        return hipErrorInvalidValue;
    const int lb = __builtin_ctz((unsigned)block) - 5;
    const size_t cus = (size_t)device_cu_count();
    const size_t ve = dtype == 0 ? 4 : 8;
    const size_t tiles = (a.count + 64 * ve - 1) / (64 * ve);     // 16-byte-lane tiles
    const bool narrow = dtype == 1 && block <= 256 && tiles <= 8 * cus;
    const bool medium = !narrow && tiles <= 16 * cus;
    dim3 grid, blk;
    AllreduceLpArgs arg = a;
    arg.xcd_ranges = narrow ? 1 : 0;
    LpFn fn;
    if (narrow) {
        const size_t tiles8 = (a.count + 64 * 4 - 1) / (64 * 4);
        launch_geometry(tiles8 * kWave, true, policy_lp_narrow(), grid, blk);
        // a message of whole tiles (of 256 elements): one tile per wave, no loop
        const bool one = a.count % (64 * 4) == 0;
        const auto& nt = fmt == 0 ? kLpB16E4Narrow.one : kLpB16E5Narrow.one;
        const auto& nr = fmt == 0 ? kLpB16E4Narrow.row : kLpB16E5Narrow.row;
        fn = one ? nt[lb][nsrc - 1] : nr[lb][nsrc - 1];
    } else {
        launch_geometry(tiles * kWave, false, medium ? policy_lp_medium() : policy_lp_large(), grid, blk);
        fn = dtype == 0 ? (fmt == 0 ? kLpF32E4.row[lb][nsrc - 1] : kLpF32E5.row[lb][nsrc - 1])
                        : (fmt == 0 ? kLpB16E4.row[lb][nsrc - 1] : kLpB16E5.row[lb][nsrc - 1]);
    }
    void* params[] = {&arg};
    return launch_logged(narrow ? "k_allreduce_lp (8-byte lanes)" : medium ? "k_allreduce_lp (medium)" : "k_allreduce_lp",
                         (const void*)fn, grid, blk, params, s);
}

}  // namespace rx
