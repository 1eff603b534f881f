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

// Widen a 16-byte vector to kVE floats (exact).
template <int DT>
__device__ __forceinline__ void widen_vec(const u32x4& x, float* f)
{
    if constexpr (DT == 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) f[k] = bits_f32(x[k]);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            f[2 * k] = bf16_lo(x[k]);
            f[2 * k + 1] = bf16_hi(x[k]);
        }
    }
}

// Elements [e, count) of a partial vector, the rest zero (neutral for the
// block absmax; never stored).
template <int DT>
__device__ __forceinline__ u32x4 load_tail(const void* src, size_t e, size_t count)
{
    u32x4 x = {0u, 0u, 0u, 0u};
    if constexpr (DT == 0) {
        const uint32_t* p = static_cast<const uint32_t*>(src);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (e + k < count) x[k] = p[e + k];
    } else {
        const uint16_t* p = static_cast<const uint16_t*>(src);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (e + k < count) x[k / 2] |= (uint32_t)p[e + k] << (16 * (k & 1));
    }
    return x;
}

// dequant(quant(f)) of the VE values of one lane, for a block whose absmax
// over its LPB lanes is taken here: out[k] = fl32(decode(code_k) * s).
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
    for (int q = 0; q < VE / 4; ++q) {
        const uint32_t w = f32x4_to_fp8<F>(clamp_fmax<F>(f[4 * q] * r), clamp_fmax<F>(f[4 * q + 1] * r),
                                           clamp_fmax<F>(f[4 * q + 2] * r), clamp_fmax<F>(f[4 * q + 3] * r));
        float d[4];
        fp8x4_to_f32<F>(w, d);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            out[4 * q + k] = d[k] * s;
    }
}

// One wave per tile of 64 vectors of every rank (lane l: vector tile * 64 +
// l); a block spans LPB = BLOCK / VE <= 64 lanes of one tile.
template <int DT, int F, int BLOCK, int N>
__global__ __launch_bounds__(256) void k_allreduce_lp(AllreduceLpArgs a)
{
    constexpr int VE = DT == 0 ? 4 : 8;
    constexpr int LPB = BLOCK / VE;
    static_assert(LPB >= 1 && LPB <= kWave, "a block lies in the lanes of one wave");
    constexpr size_t kTileElems = (size_t)kWave * VE;
    const int lane = lane_id();
    const uint32_t wave_in_wg = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t waves_per_wg = blockDim.x / kWave;
    const uint32_t wg = a.xcd_ranges ? xcd_contiguous(blockIdx.x, gridDim.x) : blockIdx.x;
    const size_t wave = (size_t)wg * waves_per_wg + wave_in_wg;
    const size_t nwaves = (size_t)gridDim.x * waves_per_wg;
    const size_t ntiles = (a.count + kTileElems - 1) / kTileElems;

    for (size_t t = wave; t < ntiles; t += nwaves) {
        const size_t v = t * kWave + lane;
        const size_t e = v * VE;
        const bool full = (t + 1) * kTileElems <= a.count;   // uniform
        u32x4 x[N];
        if (full) {
#pragma unroll
            for (int r = 0; r < N; ++r)
                x[r] = ld16_stream(a.buf[r], v);
        } else {
#pragma unroll
            for (int r = 0; r < N; ++r)
                x[r] = e + VE <= a.count ? ld16(a.buf[r], v) : load_tail<DT>(a.buf[r], e, a.count);
        }

        // every rank's block quantized and dequantized, folded in rank order
        float S[VE];
        {
            float f[VE];
            widen_vec<DT>(x[0], f);
            quant_dequant<F, LPB, VE>(f, S);
        }
#pragma unroll
        for (int r = 1; r < N; ++r) {
            float f[VE], d[VE];
            widen_vec<DT>(x[r], f);
            quant_dequant<F, LPB, VE>(f, d);
#pragma unroll
            for (int k = 0; k < VE; ++k)
                S[k] = S[k] + d[k];
        }
        // the requantized sum, dequantized: every rank's result
        float h[VE];
        quant_dequant<F, LPB, VE>(S, h);
        u32x4 y;
        if constexpr (DT == 0) {
#pragma unroll
            for (int k = 0; k < 4; ++k) y[k] = __builtin_bit_cast(uint32_t, h[k]);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) y[k] = pack_bf16(h[2 * k], h[2 * k + 1]);
        }
        if (full) {
#pragma unroll
            for (int r = 0; r < N; ++r)
                st16_stream(a.buf[r], v, y);
        } else if (e + VE <= a.count) {
#pragma unroll
            for (int r = 0; r < N; ++r)
                st16(a.buf[r], v, y);
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
    }
}

using LpFn = void (*)(AllreduceLpArgs);

template <int DT, int F, int BLOCK, int... I>
constexpr std::array<LpFn, sizeof...(I)> lp_row(std::integer_sequence<int, I...>)
{
    return {{&k_allreduce_lp<DT, F, BLOCK, I + 1>...}};
}

// Rows by block size (32, 64, ...): blocks of at most 64 vectors, FP32
// 32..256 and BF16 32..512 (larger blocks use the two-pass path).
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
    t.row[0] = lp_row<DT, F, 32>(seq);
    t.row[1] = lp_row<DT, F, 64>(seq);
    t.row[2] = lp_row<DT, F, 128>(seq);
    t.row[3] = lp_row<DT, F, 256>(seq);
    if constexpr (DT == 1)
        t.row[4] = lp_row<DT, F, 512>(seq);
    return t;
}

const LpTable<0, 0> kLpF32E4 = make_lp_table<0, 0>();
const LpTable<0, 1> kLpF32E5 = make_lp_table<0, 1>();
const LpTable<1, 0> kLpB16E4 = make_lp_table<1, 0>();
const LpTable<1, 1> kLpB16E5 = make_lp_table<1, 1>();

// Decode-size messages: one tile per wave in 64-thread workgroups over every
// CU, each XCD a contiguous range. Large ones: four 64-thread workgroups per
// CU (one wave per SIMD), grid-stride; measured on MI355X against 2-16 per
// CU and 128/256-thread workgroups: 8 x 512 MiB BF16 E5M2/256 1487 us
// (two 256-thread workgroups: 1942 us; five or three 64-thread ones: 1691,
// 1879 us), 8 x 64 MiB FP32 E4M3/128 180 us (207 us).
LaunchPolicy policy_lp() { return {64u, 64u, 4u}; }

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
    const size_t ve = dtype == 0 ? 4 : 8;
    const size_t tiles = (a.count + 64 * ve - 1) / (64 * ve);
    const bool small = tiles < kSmallTilesPerCu * (size_t)device_cu_count();
    dim3 grid, blk;
    launch_geometry(tiles * kWave, small, policy_lp(), grid, blk);
    AllreduceLpArgs arg = a;
    arg.xcd_ranges = small ? 1 : 0;
    void* params[] = {&arg};
    const LpFn fn = dtype == 0 ? (fmt == 0 ? kLpF32E4.row[lb][nsrc - 1] : kLpF32E5.row[lb][nsrc - 1])
                               : (fmt == 0 ? kLpB16E4.row[lb][nsrc - 1] : kLpB16E5.row[lb][nsrc - 1]);
    return launch_logged(small ? "k_allreduce_lp (decode size)" : "k_allreduce_lp",
                         (const void*)fn, grid, blk, params, s);
}

}  // namespace rx
