// quant.hip -- FP32/BF16 -> OCP FP8 block quantizer on gfx950, the sender
// side of the low-precision collectives (RCCLX article, code-journey.com,
// "Core feature 2: Low-Precision Collectives": FP8 quantization with up to
// 4:1 compression; table row "Data types").
//
// Encoding (a reading; the pages give only "FP8"): one FP32 scale per block
// of B elements, s = A / FMAX with A the block absmax; elements multiplied
// by r = FMAX / A, clamped to +-FMAX and converted with round-to-nearest-even
// on the hardware converters (v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32).
//
// One streaming pass with no LDS: every load is a coalesced 16-byte load
// (lane l of a wave reads vector base + l), the block absmax is reduced
// across the lanes that hold the block with DPP and permlane swaps, and each
// lane stores its own codes.
#include <array>
#include <utility>

#include "rx_device.hpp"
#include "rx_internal.hpp"

namespace rx {
namespace {

// ---------------------------------------------------------------------------
// Quantizer
// ---------------------------------------------------------------------------

// A wave processes tiles of U loads per lane (U x 1 KiB per tile): U = 4 or 8
// for large messages (8 with the next tile's loads in flight; launch_quant
// picks by size), U = the loads per block (usually 1) for decode-size
// messages (4x the waves, shorter serial chains).
template <int DT, int F, int BLOCK, int U>
struct QuantShape {
    static constexpr int kVE = DT == 0 ? 4 : 8;          // elements per 16-B vector
    static constexpr int kLanesRaw = BLOCK / kVE;        // vectors per block
    static constexpr int kLPB = kLanesRaw < 64 ? kLanesRaw : 64;  // lanes per block
    static constexpr int kUPB = kLanesRaw / kLPB;        // loads per block (1, 2, 4)
    static constexpr int kU = U;                         // loads per lane per tile
    static constexpr int kTileVec = kWave * kU;
    static constexpr int kTileElems = kTileVec * kVE;
    static_assert(kU % kUPB == 0, "a tile holds whole blocks");
    static_assert(kLanesRaw >= 1, "block of at least one vector");
};

template <int DT, int BLOCK>
constexpr int loads_per_block()
{
    constexpr int lanes = BLOCK / (DT == 0 ? 4 : 8);
    return lanes <= 64 ? 1 : lanes / 64;
}

// Widen vector x (16 bytes) to kVE floats.
template <int DT>
__device__ __forceinline__ void widen(const u32x4& x, float* f)
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

// Partial vector at the end of a ragged source: elements [e, count), the
// rest zero (zero is neutral for the absmax). Every element is loaded from
// an index clamped to count - 1 (in bounds, count >= 1) and masked
// afterwards, so the loads carry no branches and are all in flight before
// the first use.
template <int DT>
__device__ __forceinline__ u32x4 load_partial(const void* src, size_t e, size_t count)
{
    u32x4 x = {0u, 0u, 0u, 0u};
    if constexpr (DT == 0) {
        const uint32_t* p = static_cast<const uint32_t*>(src);
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            w[k] = p[e + k < count ? e + k : count - 1];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            x[k] = e + k < count ? w[k] : 0u;
    } else {
        const uint16_t* p = static_cast<const uint16_t*>(src);
        uint32_t h[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            h[k] = p[e + k < count ? e + k : count - 1];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            x[k / 2] |= (e + k < count ? h[k] : 0u) << (16 * (k & 1));
    }
    return x;
}

// Codes and block scales of one tile (x: the U loads of this lane, vector
// v0 + u * 64 + lane). full: every element of the tile lies inside the
// source; otherwise the codes and scales past count are not stored. SMALL:
// scales stored nontemporal (decode-size launches).
template <int DT, int F, int BLOCK, int U, bool SMALL>
__device__ __forceinline__ void quant_tile(const u32x4 (&x)[U], uint8_t* codes, float* scales, size_t v0,
                                           size_t count, bool full, int lane)
{
    using Sh = QuantShape<DT, F, BLOCK, U>;
    constexpr int VE = Sh::kVE, LPB = Sh::kLPB, UPB = Sh::kUPB;
    float f[U][VE];
    float amax[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        widen<DT>(x[u], f[u]);
        float m = __builtin_fabsf(f[u][0]);
#pragma unroll
        for (int k = 1; k < VE; ++k)
            m = __builtin_fmaxf(m, __builtin_fabsf(f[u][k]));
        amax[u] = m;
    }

    // Block absmax across the lanes (and loads) that hold the block.
    float s[U], r[U];
    if constexpr (UPB == 1) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float A = bits_f32(group_max<LPB>(__builtin_bit_cast(uint32_t, amax[u])));
            block_scale<F>(A, s[u], r[u]);
        }
    } else {
#pragma unroll
        for (int g = 0; g < U / UPB; ++g) {
            float m = amax[g * UPB];
#pragma unroll
            for (int q = 1; q < UPB; ++q)
                m = __builtin_fmaxf(m, amax[g * UPB + q]);
            float A = bits_f32(group_max<64>(__builtin_bit_cast(uint32_t, m)));
            float sg, rg;
            block_scale<F>(A, sg, rg);
#pragma unroll
            for (int q = 0; q < UPB; ++q) {
                s[g * UPB + q] = sg;
                r[g * UPB + q] = rg;
            }
        }
    }

    // Encode and store: VE codes per lane per load (4 or 8 bytes).
#pragma unroll
    for (int u = 0; u < U; ++u) {
        uint32_t w[VE / 4];
#pragma unroll
        for (int q = 0; q < VE / 4; ++q) {
            float y0 = clamp_fmax<F>(f[u][4 * q + 0] * r[u]);
            float y1 = clamp_fmax<F>(f[u][4 * q + 1] * r[u]);
            float y2 = clamp_fmax<F>(f[u][4 * q + 2] * r[u]);
            float y3 = clamp_fmax<F>(f[u][4 * q + 3] * r[u]);
            w[q] = f32x4_to_fp8<F>(y0, y1, y2, y3);
        }
        const size_t vi = v0 + u * kWave + lane;
        const size_t e = vi * VE;
        if (full || e + VE <= count) {
            // contiguous across the wave: stream past the caches
            if constexpr (VE == 4) {
                __builtin_nontemporal_store(w[0], reinterpret_cast<uint32_t*>(codes) + vi);
            } else {
                u32x2 p = {w[0], w[1]};
                __builtin_nontemporal_store(p, reinterpret_cast<u32x2*>(codes) + vi);
            }
        } else {
#pragma unroll
            for (int k = 0; k < VE; ++k)
                if (e + k < count)
                    codes[e + k] = (uint8_t)(w[k / 4] >> (8 * (k & 3)));
        }
        // one lane per block writes the scale
        const bool leader = UPB == 1 ? (lane % LPB) == 0 : (lane == 0 && u % UPB == 0);
        if (leader && (full || e < count)) {
            if constexpr (SMALL)
                __builtin_nontemporal_store(s[u], scales + e / BLOCK);
            else
                scales[e / BLOCK] = s[u];
        }
    }
}

// Any message, tiles that may end past the source (decode-size launches and
// the ragged ends of large ones). SMALL (decode size, one tile per wave):
// each XCD takes a contiguous range of tiles and the block scales are stored
// nontemporal, so that no line of scales is left partly written in several
// L2s for the end-of-kernel write-back (together 7% faster at 8 x 512 KiB;
// at large sizes both were slower, up to 13%, and the scale lines fill up in
// L2 instead).
template <int DT, int F, int BLOCK, int UL, bool SMALL>
__global__ __launch_bounds__(256) void k_quant(QuantArgs a)
{
    using Sh = QuantShape<DT, F, BLOCK, UL>;
    constexpr int VE = Sh::kVE, U = Sh::kU;
    const int lane = lane_id();
    const uint32_t wave_in_wg = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t waves_per_wg = blockDim.x / kWave;
    const uint32_t wg = SMALL ? xcd_contiguous(blockIdx.x, gridDim.x) : blockIdx.x;
    const uint32_t wave = wg * waves_per_wg + wave_in_wg;
    const uint32_t nwaves = gridDim.x * waves_per_wg;
    const uint32_t tiles_per_src = (uint32_t)((a.count + Sh::kTileElems - 1) / Sh::kTileElems);
    const uint32_t total = tiles_per_src * (uint32_t)a.nsrc;

    for (uint32_t t = wave; t < total; t += nwaves) {
        const uint32_t j = t / tiles_per_src;
        const uint32_t tile = t - j * tiles_per_src;
        const void* src = a.src[j];
        const size_t e0 = (size_t)tile * Sh::kTileElems;   // first element of the tile
        const size_t v0 = e0 / VE;
        const bool full = e0 + Sh::kTileElems <= a.count;

        u32x4 x[U];
        if (full) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                x[u] = ld16_stream(src, v0 + u * kWave + lane);
        } else {
            // the partial last tile of a source: element loads, no branches
#pragma unroll
            for (int u = 0; u < U; ++u)
                x[u] = load_partial<DT>(src, (v0 + u * kWave + lane) * VE, a.count);
        }
        quant_tile<DT, F, BLOCK, U, SMALL>(x, static_cast<uint8_t*>(a.codes[j]), a.scales[j], v0, a.count,
                                           full, lane);
    }
}

// Decode-size messages whose sources are whole tiles (count a multiple of
// the tile): one tile per wave and no loop, nontemporal scale stores (as
// k_quant's SMALL instances, without the grid-stride loop and the
// partial-tile path: 8 x 256K BF16 E5M2/256 3.12 -> 3.07 us). One row of
// 256-thread workgroups per source (blockIdx.y), quant_tile_row(tiles)
// workgroups wide: a multiple of 8, so workgroup x of every row runs on XCD
// x % 8 and each XCD owns a contiguous range of the row's tiles. No division
// maps a tile to its source, and the exit test reads the source's pointers,
// so every kernel-argument load is issued at once, before the first branch,
// and the tile's loads wait for one scalar round trip (8 x 256K BF16 3.05 ->
// 2.88 us, 8 x 512K BF16 4.44 -> 3.76, 8 x 37 tiles 2.54 -> 2.05, 8 x 1001
// tiles FP32 E4M3/128 4.23 -> 3.68, against a 1-D grid of all sources'
// tiles).
constexpr uint32_t kQuantTileWaves = 4;

__host__ __device__ constexpr uint32_t quant_tile_row(uint32_t tiles)
{
    return ((tiles + kQuantTileWaves - 1) / kQuantTileWaves + kXcds - 1) / kXcds * kXcds;
}

template <int DT, int F, int BLOCK, int UL>
__global__ __launch_bounds__(256) void k_quant_tile(QuantArgs a)
{
    using Sh = QuantShape<DT, F, BLOCK, UL>;
    constexpr int U = Sh::kU;
    const uint32_t j = blockIdx.y;
    const void* src = a.src[j];
    uint8_t* codes = static_cast<uint8_t*>(a.codes[j]);
    float* scales = a.scales[j];
    const size_t count = a.count;
    const int lane = lane_id();
    const uint32_t wave_in_wg = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t tiles = (uint32_t)(count / Sh::kTileElems);
    const uint32_t t = xcd_contiguous(blockIdx.x, quant_tile_row(tiles)) * kQuantTileWaves + wave_in_wg;
    if (t >= tiles || src == nullptr || codes == nullptr || scales == nullptr)
        return;
    const size_t v0 = (size_t)t * Sh::kTileVec;
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        x[u] = ld16_stream(src, v0 + u * kWave + lane);
    quant_tile<DT, F, BLOCK, U, true>(x, codes, scales, v0, count, true, lane);
}

// The U loads of tile t (tile t % tiles_per_src of source t / tiles_per_src).
template <int DT, int F, int BLOCK, int U>
__device__ __forceinline__ void load_whole_tile(u32x4 (&x)[U], const QuantArgs& a, uint32_t t,
                                                uint32_t tiles_per_src, int lane)
{
    using Sh = QuantShape<DT, F, BLOCK, U>;
    const uint32_t j = t / tiles_per_src;
    const size_t v0 = (size_t)(t - j * tiles_per_src) * Sh::kTileVec;
#pragma unroll
    for (int u = 0; u < U; ++u)
        x[u] = ld16_stream(a.src[j], v0 + u * kWave + lane);
}

template <int DT, int F, int BLOCK, int U>
__device__ __forceinline__ void quant_whole_tile(const u32x4 (&x)[U], const QuantArgs& a, uint32_t t,
                                                 uint32_t tiles_per_src, int lane)
{
    using Sh = QuantShape<DT, F, BLOCK, U>;
    const uint32_t j = t / tiles_per_src;
    const size_t v0 = (size_t)(t - j * tiles_per_src) * Sh::kTileVec;
    quant_tile<DT, F, BLOCK, U, false>(x, static_cast<uint8_t*>(a.codes[j]), a.scales[j], v0, a.count, true,
                                       lane);
}

// Large messages, whole tiles only (count a multiple of the tile; the ragged
// end of each source goes to k_quant). Without the partial-tile code the
// kernel ran 6% faster (8 x 16M FP32 E4M3/128: 112.6 -> 106.0 us). PF: the
// next tile's loads are issued before this tile's arithmetic, into the other
// of two register buffers; the last tile of a wave is peeled off, so that in
// the loop every prefetch is unconditional and the compiler waits only for
// the current tile's loads (8 x 256M BF16 E5M2/256: 1148 -> 1073 us, at one
// 256-thread workgroup per CU).
template <int DT, int F, int BLOCK, int U, bool PF>
__global__ __launch_bounds__(256) void k_quant_whole(QuantArgs a)
{
    using Sh = QuantShape<DT, F, BLOCK, U>;
    const int lane = lane_id();
    const uint32_t wave_in_wg = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t wave = blockIdx.x * (blockDim.x / kWave) + wave_in_wg;
    const uint32_t nwaves = gridDim.x * (blockDim.x / kWave);
    const uint32_t tiles_per_src = (uint32_t)(a.count / Sh::kTileElems);
    const uint32_t total = tiles_per_src * (uint32_t)a.nsrc;
    uint32_t t = wave;
    if (t >= total)
        return;
    if constexpr (PF) {
        u32x4 xa[U], xb[U];
        uint32_t n = (total - t + nwaves - 1) / nwaves;   // tiles of this wave, >= 1
        load_whole_tile<DT, F, BLOCK, U>(xa, a, t, tiles_per_src, lane);
        for (;;) {
            if (n == 1) {
                quant_whole_tile<DT, F, BLOCK, U>(xa, a, t, tiles_per_src, lane);
                break;
            }
            load_whole_tile<DT, F, BLOCK, U>(xb, a, t + nwaves, tiles_per_src, lane);
            quant_whole_tile<DT, F, BLOCK, U>(xa, a, t, tiles_per_src, lane);
            t += nwaves;
            --n;
            if (n == 1) {
                quant_whole_tile<DT, F, BLOCK, U>(xb, a, t, tiles_per_src, lane);
                break;
            }
            load_whole_tile<DT, F, BLOCK, U>(xa, a, t + nwaves, tiles_per_src, lane);
            quant_whole_tile<DT, F, BLOCK, U>(xb, a, t, tiles_per_src, lane);
            t += nwaves;
            --n;
        }
    } else {
        for (; t < total; t += nwaves) {
            u32x4 x[U];
            load_whole_tile<DT, F, BLOCK, U>(x, a, t, tiles_per_src, lane);
            quant_whole_tile<DT, F, BLOCK, U>(x, a, t, tiles_per_src, lane);
        }
    }
}

using QuantFn = void (*)(QuantArgs);

// Decode-size variants: U = the loads per block.
template <int DT, int F, int... L>
constexpr std::array<QuantFn, sizeof...(L)> quant_row(std::integer_sequence<int, L...>)
{
    return {{&k_quant<DT, F, (32 << L), loads_per_block<DT, (32 << L)>(), true>...}};
}
template <int DT, int F, int... L>
constexpr std::array<QuantFn, sizeof...(L)> quant_tile_row(std::integer_sequence<int, L...>)
{
    return {{&k_quant_tile<DT, F, (32 << L), loads_per_block<DT, (32 << L)>()>...}};
}

template <int DT, int F, int U, bool PF, int... L>
constexpr std::array<QuantFn, sizeof...(L)> quant_whole_row(std::integer_sequence<int, L...>)
{
    return {{&k_quant_whole<DT, F, (32 << L), U, PF>...}};
}

// [src dtype][fmt][log2(block) - 5]
struct QuantTable {
    std::array<QuantFn, 6> fn[2][2] = {
        {quant_row<0, 0>(std::make_integer_sequence<int, 6>{}), quant_row<0, 1>(std::make_integer_sequence<int, 6>{})},
        {quant_row<1, 0>(std::make_integer_sequence<int, 6>{}), quant_row<1, 1>(std::make_integer_sequence<int, 6>{})}};
};
template <int U, bool PF>
struct QuantWholeTable {
    std::array<QuantFn, 6> fn[2][2] = {
        {quant_whole_row<0, 0, U, PF>(std::make_integer_sequence<int, 6>{}),
         quant_whole_row<0, 1, U, PF>(std::make_integer_sequence<int, 6>{})},
        {quant_whole_row<1, 0, U, PF>(std::make_integer_sequence<int, 6>{}),
         quant_whole_row<1, 1, U, PF>(std::make_integer_sequence<int, 6>{})}};
};
struct QuantTileTable {
    std::array<QuantFn, 6> fn[2][2] = {
        {quant_tile_row<0, 0>(std::make_integer_sequence<int, 6>{}),
         quant_tile_row<0, 1>(std::make_integer_sequence<int, 6>{})},
        {quant_tile_row<1, 0>(std::make_integer_sequence<int, 6>{}),
         quant_tile_row<1, 1>(std::make_integer_sequence<int, 6>{})}};
};
const QuantTable kQuantSmall;
const QuantTileTable kQuantTile;
const QuantWholeTable<4, false> kQuantWhole4;
const QuantWholeTable<8, true> kQuantWhole8Pf;

// One wave per tile (64 threads per work item), 256-thread workgroups.
LaunchPolicy policy_quant() { return {256u, 256u, 2u}; }

// Decode-size kernel over any message: one tile (one block's loads) per wave
// over every CU.
hipError_t launch_quant_tiles(const QuantArgs& a, int src_dtype, int fmt, int block, hipStream_t s)
{
    const int lb = __builtin_ctz((unsigned)block) - 5;
    const size_t vec_elems = src_dtype == 0 ? 4 : 8;
    const size_t lanes_per_block = (size_t)block / vec_elems;
    const size_t u = lanes_per_block <= 64 ? 1 : lanes_per_block / 64;
    const size_t tile_elems = u * 64 * vec_elems;
    QuantArgs arg = a;
    void* params[] = {&arg};
    if (a.count % tile_elems == 0) {
        // sources of whole tiles: the loop-free kernel, one row per source
        const size_t tiles = a.count / tile_elems;
        if (tiles > 0xFFFFFFFFull / kQuantTileWaves)
            return hipErrorInvalidConfiguration;
        const dim3 grid(quant_tile_row((uint32_t)tiles), (unsigned)a.nsrc);
        const dim3 blk(kQuantTileWaves * kWave);
        return launch_logged("k_quant_tile (decode size)", (const void*)kQuantTile.fn[src_dtype][fmt][lb], grid, blk,
                             params, s);
    }
    const size_t tiles = (a.count + tile_elems - 1) / tile_elems * (size_t)a.nsrc;
    dim3 grid, blk;
    launch_geometry(tiles * kWave, true, policy_quant(), grid, blk);
    return launch_logged("k_quant (decode size)", (const void*)kQuantSmall.fn[src_dtype][fmt][lb], grid, blk,
                         params, s);
}

}  // namespace

hipError_t launch_quant(const QuantArgs& a, int src_dtype, int fmt, int block, hipStream_t s)
{
    const int lb = __builtin_ctz((unsigned)block) - 5;
    const size_t vec_elems = src_dtype == 0 ? 4 : 8;
    const size_t cus = (size_t)device_cu_count();
    const size_t large_tiles = (a.count + 4 * 64 * vec_elems - 1) / (4 * 64 * vec_elems) * (size_t)a.nsrc;
    if (large_tiles < kSmallTilesPerCu * cus)
        return launch_quant_tiles(a, src_dtype, fmt, block, s);
    // Sources of whole decode-size tiles up to 16 (BF16) or 8 (FP32) of the
    // tiles below per CU: the loop-free kernel, a wave per tile (8 sources:
    // 8 x 512K BF16 E5M2/256 4.20 -> 3.75 us, 8 x 1M 6.67 -> 6.28, 8 x 256K
    // FP32 E4M3/128 3.87 -> 3.72; at 32 per CU and above BF16 gained 0-3.5%
    // and FP32 lost 7-23%, so they stay below)
    const size_t lanes_per_block = (size_t)block / vec_elems;
    const size_t decode_tile = (lanes_per_block <= 64 ? 1 : lanes_per_block / 64) * 64 * vec_elems;
    if (a.count % decode_tile == 0 && large_tiles <= (src_dtype == 0 ? 8 : 16) * cus)
        return launch_quant_tiles(a, src_dtype, fmt, block, s);
    dim3 grid, blk;
    // Large messages: whole tiles in k_quant_whole, then the ragged end of
    // each source (less than one tile) in the decode-size kernel. A tile of
    // 4 loads per lane is 4 KiB of input. From 4 MiB of input per CU
    // (1024 such tiles): 8 loads per lane with the next tile prefetched, one
    // workgroup per CU (8 x 256M BF16 E5M2/256 1080 us against 1157 us for
    // 4 loads at two per CU; 8 x 64M BF16 259.5 against 265.2 us, FP32
    // 435.5 against 438.1 us); below: 4 loads per lane, two workgroups per
    // CU (8 x 16M FP32 E4M3/128 106.4 us against 109.4 us with the
    // prefetch), four below 64 tiles per CU (8 x 1M FP32 8.8 against
    // 9.1 us).
    const bool pf = large_tiles >= (size_t)1024 * cus;
    const size_t u = pf ? 8 : 4;
    const size_t tile_elems = u * 64 * vec_elems;
    const size_t whole = a.count / tile_elems;
    if (whole) {
        LaunchPolicy pol = policy_quant();
        pol.max_wgs_per_cu = pf ? 1 : large_tiles < (size_t)64 * cus ? 4 : 2;
        launch_geometry(whole * (size_t)a.nsrc * kWave, false, pol, grid, blk);
        QuantArgs arg = a;
        arg.count = whole * tile_elems;
        void* params[] = {&arg};
        const QuantFn fn = pf ? kQuantWhole8Pf.fn[src_dtype][fmt][lb] : kQuantWhole4.fn[src_dtype][fmt][lb];
        const hipError_t e = launch_logged(pf ? "k_quant_whole (8 loads, prefetch)" : "k_quant_whole", (const void*)fn,
                                           grid, blk, params, s);
        if (e != hipSuccess)
            return e;
    }
    if (a.count % tile_elems == 0)
        return hipSuccess;
    // tile_elems is a multiple of the block, so the rest starts on a block
    QuantArgs rest = a;
    const size_t done = whole * tile_elems;
    for (int j = 0; j < a.nsrc; ++j) {
        rest.src[j] = static_cast<const uint8_t*>(a.src[j]) + done * (src_dtype == 0 ? 4 : 2);
        rest.codes[j] = static_cast<uint8_t*>(a.codes[j]) + done;
        rest.scales[j] = a.scales[j] + done / (size_t)block;
    }
    rest.count = a.count - done;
    return launch_quant_tiles(rest, src_dtype, fmt, block, s);
}

}  // namespace rx
