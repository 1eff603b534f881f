// lowprec.hip -- the low-precision collective path on gfx950: FP32/BF16 ->
// OCP FP8 block quantizer, and the fused dequantize -> FP32 sum ->
// requantize step (RCCLX article, code-journey.com, "Core feature 2:
// Low-Precision Collectives": FP8 quantization with up to 4:1 compression,
// FP32 compute; table rows "Data types" and "Compute precision").
//
// Encoding (a reading; the pages give only "FP8"): one FP32 scale per block
// of B elements, s = A / FMAX with A the block absmax; elements multiplied
// by r = FMAX / A, clamped to +-FMAX and converted with round-to-nearest-even
// on the hardware converters (v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32).
//
// Both kernels are single streaming passes with no LDS: every load is a
// coalesced 16-byte load (lane l of a wave reads vector base + l), the block
// absmax is reduced across the lanes that hold the block with DPP and
// permlane swaps, and each lane stores its own codes.
#include <array>
#include <utility>

#include "rx_device.hpp"
#include "rx_internal.hpp"

namespace rx {
namespace {

// ---------------------------------------------------------------------------
// Quantizer
// ---------------------------------------------------------------------------

// A wave processes tiles of U loads per lane (U x 1 KiB per tile): U = 4 for
// large messages (more bytes in flight per wave), U = the loads per block
// (usually 1) for decode-size messages (4x the waves, shorter serial chains).
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

// Partial vector at the end of a ragged source: elements [e, count) loaded
// one by one, the rest zero (zero is neutral for the absmax).
template <int DT>
__device__ __forceinline__ u32x4 load_partial(const void* src, size_t e, size_t count)
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

template <int DT, int F, int BLOCK, int UL>
__global__ __launch_bounds__(256) void k_quant(QuantArgs a)
{
    using Sh = QuantShape<DT, F, BLOCK, UL>;
    constexpr int VE = Sh::kVE, U = Sh::kU, LPB = Sh::kLPB, UPB = Sh::kUPB;
    const int lane = lane_id();
    const uint32_t wave_in_wg = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t waves_per_wg = blockDim.x / kWave;
    const uint32_t wave = blockIdx.x * waves_per_wg + wave_in_wg;
    const uint32_t nwaves = gridDim.x * waves_per_wg;
    const uint32_t tiles_per_src = (uint32_t)((a.count + Sh::kTileElems - 1) / Sh::kTileElems);
    const uint32_t total = tiles_per_src * (uint32_t)a.nsrc;

    for (uint32_t t = wave; t < total; t += nwaves) {
        const uint32_t j = t / tiles_per_src;
        const uint32_t tile = t - j * tiles_per_src;
        const void* src = a.src[j];
        uint8_t* codes = static_cast<uint8_t*>(a.codes[j]);
        float* scales = a.scales[j];
        const size_t e0 = (size_t)tile * Sh::kTileElems;   // first element of the tile
        const size_t v0 = e0 / VE;
        const bool full = e0 + Sh::kTileElems <= a.count;

        u32x4 x[U];
        if (full) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                x[u] = ld16_stream(src, v0 + u * kWave + lane);
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const size_t e = (v0 + u * kWave + lane) * VE;
                if (e + VE <= a.count)
                    x[u] = ld16(src, v0 + u * kWave + lane);
                else
                    x[u] = load_partial<DT>(src, e, a.count);
            }
        }

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
            if (full || e + VE <= a.count) {
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
                    if (e + k < a.count)
                        codes[e + k] = (uint8_t)(w[k / 4] >> (8 * (k & 3)));
            }
            // one lane per block writes the scale
            const bool leader = UPB == 1 ? (lane % LPB) == 0 : (lane == 0 && u % UPB == 0);
            if (leader && e < a.count)
                scales[e / BLOCK] = s[u];
        }
    }
}

// ---------------------------------------------------------------------------
// Dequantize -> FP32 sum -> (requantize)
// ---------------------------------------------------------------------------

// Lane layout of a wave tile of 64 * CPC * U codes: lane l owns U chunks of
// CPC consecutive codes, chunk u at tile offset (u * 64 + l) * CPC. Every
// load and store instruction then covers one contiguous run (64 lanes x CPC
// codes, or their 2- or 4-byte outputs). Layouts used:
//   CPC 16, U 1: dwordx4 code loads (any block size);
//   CPC  8, U 2: BF16 output, 16-byte stores contiguous across the wave;
//   CPC  4, U 4: FP32 output, 16-byte stores contiguous across the wave;
//   CPC  4, U 1: decode-size messages (4x the waves, short serial chains).
// A block spans block / CPC lanes of one chunk; the launcher only picks
// layouts with block / CPC <= 64.
template <int CPC>
struct Chunk {
    uint32_t w[CPC / 4];
};

template <int CPC>
__device__ __forceinline__ Chunk<CPC> load_chunk(const uint8_t* p, size_t c, size_t e,
                                                 size_t count, bool whole)
{
    Chunk<CPC> x;
    if (whole) {
        if constexpr (CPC == 16) {
            u32x4 v = ld16_stream(p, c);
#pragma unroll
            for (int q = 0; q < 4; ++q) x.w[q] = v[q];
        } else if constexpr (CPC == 8) {
            u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p) + c);
            x.w[0] = v[0];
            x.w[1] = v[1];
        } else {
            x.w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p) + c);
        }
    } else {  // codes [e, count) byte by byte, the rest code 0 (decodes to +0)
#pragma unroll
        for (int q = 0; q < CPC / 4; ++q) x.w[q] = 0u;
#pragma unroll
        for (int k = 0; k < CPC; ++k)
            if (e + k < count) x.w[k / 4] |= (uint32_t)p[e + k] << (8 * (k & 3));
    }
    return x;
}

template <int F, int CPC>
__device__ __forceinline__ void dequant(const uint32_t* w, float sc, float* v)
{
#pragma unroll
    for (int q = 0; q < CPC / 4; ++q) {
        float d[4];
        fp8x4_to_f32<F>(w[q], d);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            v[4 * q + k] = d[k] * sc;
    }
}

// Code stores are contiguous across the wave: stream past the caches.
template <int CPC>
__device__ __forceinline__ void store_codes(uint8_t* p, size_t c, size_t e, size_t count,
                                            bool whole, const uint32_t* w)
{
    if (whole) {
        if constexpr (CPC == 16) {
            u32x4 v = {w[0], w[1], w[2], w[3]};
            st16_stream(p, c, v);
        } else if constexpr (CPC == 8) {
            u32x2 v = {w[0], w[1]};
            __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p) + c);
        } else {
            __builtin_nontemporal_store(w[0], reinterpret_cast<uint32_t*>(p) + c);
        }
    } else {
#pragma unroll
        for (int k = 0; k < CPC; ++k)
            if (e + k < count) p[e + k] = (uint8_t)(w[k / 4] >> (8 * (k & 3)));
    }
}

// High-precision values of elements e .. e + CPC - 1 (chunk c). When a lane's
// output is one 16-byte (or 8-byte) piece, the store instruction covers a
// contiguous run and streams past the caches; wider outputs are written as
// strided 16-byte pieces with cached stores, which merge in L2.
template <int CPC>
__device__ __forceinline__ void store_hp(void* out, bool bf16, size_t c, size_t e, size_t count,
                                         bool whole, const float* h)
{
    if (whole) {
        if (bf16) {
            uint32_t p[CPC / 2];
#pragma unroll
            for (int i = 0; i < CPC / 2; ++i) p[i] = pack_bf16(h[2 * i], h[2 * i + 1]);
            if constexpr (CPC == 4) {
                u32x2 v = {p[0], p[1]};
                __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(out) + c);
            } else if constexpr (CPC == 8) {
                u32x4 v = {p[0], p[1], p[2], p[3]};
                st16_stream(out, c, v);
            } else {
                u32x4 v0 = {p[0], p[1], p[2], p[3]};
                u32x4 v1 = {p[4], p[5], p[6], p[7]};
                st16(out, 2 * c, v0);
                st16(out, 2 * c + 1, v1);
            }
        } else {
#pragma unroll
            for (int q = 0; q < CPC / 4; ++q) {
                u32x4 v = {__builtin_bit_cast(uint32_t, h[4 * q]),
                           __builtin_bit_cast(uint32_t, h[4 * q + 1]),
                           __builtin_bit_cast(uint32_t, h[4 * q + 2]),
                           __builtin_bit_cast(uint32_t, h[4 * q + 3])};
                if constexpr (CPC == 4)
                    st16_stream(out, c, v);
                else
                    st16(out, (CPC / 4) * c + q, v);
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < CPC; ++k) {
            if (e + k < count) {
                if (bf16)
                    static_cast<uint16_t*>(out)[e + k] = (uint16_t)(pack_bf16(h[k], 0.0f) & 0xFFFFu);
                else
                    static_cast<float*>(out)[e + k] = h[k];
            }
        }
    }
}

// MULTI: the requantized result goes to a.nout destinations (the
// low-precision tree step's push); otherwise to out_codes[0] / out_scales[0].
template <int F, int N, bool REQUANT, int CPC, int U, bool MULTI>
__global__ __launch_bounds__(256) void k_drr(DrrArgs a)
{
    const int lane = lane_id();
    const uint32_t wave_in_wg = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t waves_per_wg = blockDim.x / kWave;
    const uint32_t wave = blockIdx.x * waves_per_wg + wave_in_wg;
    const uint32_t nwaves = gridDim.x * waves_per_wg;
    const size_t count = a.hi;                                    // end of the range
    constexpr size_t kTile = (size_t)kWave * CPC * U;             // codes per wave tile
    const uint32_t ntiles = (uint32_t)((a.hi - a.lo + kTile - 1) / kTile);
    const size_t c0 = a.lo / CPC;                                 // lo is a block multiple
    const int lpb = a.block / CPC;                                // lanes per block: <= 64
    const int bshift = __builtin_ctz((unsigned)a.block);

    for (uint32_t t = wave; t < ntiles; t += nwaves) {
        size_t c[U], e[U], b[U];
        bool whole[U], valid[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            c[u] = c0 + ((size_t)t * U + u) * kWave + lane;  // this lane's chunk u
            e[u] = c[u] * CPC;
            whole[u] = e[u] + CPC <= count;
            valid[u] = e[u] < count;
            b[u] = e[u] >> bshift;
        }

        Chunk<CPC> x[N][U];
        float sc[N][U];
#pragma unroll
        for (int r = 0; r < N; ++r) {
            const uint8_t* cp = static_cast<const uint8_t*>(a.codes[r]);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                x[r][u] = load_chunk<CPC>(cp, c[u], e[u], count, whole[u]);
                sc[r][u] = valid[u] ? a.scales[r][b[u]] : 0.0f;
            }
        }

#pragma unroll
        for (int u = 0; u < U; ++u) {
            float S[CPC];
            dequant<F, CPC>(x[0][u].w, sc[0][u], S);
#pragma unroll
            for (int r = 1; r < N; ++r) {
                float d[CPC];
                dequant<F, CPC>(x[r][u].w, sc[r][u], d);
#pragma unroll
                for (int k = 0; k < CPC; ++k)
                    S[k] = S[k] + d[k];
            }

            if constexpr (!REQUANT) {
                store_hp<CPC>(a.out_hp, a.hp_bf16 != 0, c[u], e[u], count, whole[u], S);
                continue;
            }

            // Requantize the FP32 sum with the same block size and format.
            float m = __builtin_fabsf(S[0]);
#pragma unroll
            for (int k = 1; k < CPC; ++k)
                m = __builtin_fmaxf(m, __builtin_fabsf(S[k]));
            const float A = bits_f32(group_max_rt(__builtin_bit_cast(uint32_t, m), lpb));
            float s2, r2;
            block_scale<F>(A, s2, r2);
            uint32_t q[CPC / 4];
#pragma unroll
            for (int p = 0; p < CPC / 4; ++p)
                q[p] = f32x4_to_fp8<F>(clamp_fmax<F>(S[4 * p + 0] * r2), clamp_fmax<F>(S[4 * p + 1] * r2),
                                       clamp_fmax<F>(S[4 * p + 2] * r2), clamp_fmax<F>(S[4 * p + 3] * r2));
            if constexpr (MULTI) {
                for (int j = 0; j < a.nout; ++j)   // push the chunk to every destination
                    store_codes<CPC>(static_cast<uint8_t*>(a.out_codes[j]), c[u], e[u], count, whole[u], q);
                if (valid[u] && (lane % lpb) == 0)
                    for (int j = 0; j < a.nout; ++j)
                        a.out_scales[j][b[u]] = s2;
            } else {
                store_codes<CPC>(static_cast<uint8_t*>(a.out_codes[0]), c[u], e[u], count, whole[u], q);
                if (valid[u] && (lane % lpb) == 0)
                    a.out_scales[0][b[u]] = s2;
            }

            if (a.out_hp) {
                float h[CPC];
                dequant<F, CPC>(q, s2, h);
                store_hp<CPC>(a.out_hp, a.hp_bf16 != 0, c[u], e[u], count, whole[u], h);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Dispatch tables
// ---------------------------------------------------------------------------

using QuantFn = void (*)(QuantArgs);
using DrrFn = void (*)(DrrArgs);

template <int DT, int F, bool SMALL, int... L>
constexpr std::array<QuantFn, sizeof...(L)> quant_row(std::integer_sequence<int, L...>)
{
    return {{&k_quant<DT, F, (32 << L), SMALL ? loads_per_block<DT, (32 << L)>() : 4>...}};
}

template <bool SMALL>
struct QuantTable {
    // [src dtype][fmt][log2(block) - 5]
    std::array<QuantFn, 6> fn[2][2] = {
        {quant_row<0, 0, SMALL>(std::make_integer_sequence<int, 6>{}),
         quant_row<0, 1, SMALL>(std::make_integer_sequence<int, 6>{})},
        {quant_row<1, 0, SMALL>(std::make_integer_sequence<int, 6>{}),
         quant_row<1, 1, SMALL>(std::make_integer_sequence<int, 6>{})}};
};
const QuantTable<false> kQuantLarge;
const QuantTable<true> kQuantSmall;

template <int F, bool R, int CPC, int U, bool M, int... I>
constexpr std::array<DrrFn, sizeof...(I)> drr_row(std::integer_sequence<int, I...>)
{
    return {{&k_drr<F, I + 1, R, CPC, U, M>...}};
}

template <int CPC, int U>
struct DrrTable {
    // [fmt][0 sum, 1 requant, 2 requant to every destination][nsrc - 1]
    std::array<DrrFn, kMaxSrc> fn[2][3] = {
        {drr_row<0, false, CPC, U, false>(std::make_integer_sequence<int, kMaxSrc>{}),
         drr_row<0, true, CPC, U, false>(std::make_integer_sequence<int, kMaxSrc>{}),
         drr_row<0, true, CPC, U, true>(std::make_integer_sequence<int, kMaxSrc>{})},
        {drr_row<1, false, CPC, U, false>(std::make_integer_sequence<int, kMaxSrc>{}),
         drr_row<1, true, CPC, U, false>(std::make_integer_sequence<int, kMaxSrc>{}),
         drr_row<1, true, CPC, U, true>(std::make_integer_sequence<int, kMaxSrc>{})}};
};
const DrrTable<16, 1> kDrr16x1;
const DrrTable<8, 2> kDrr8x2;
const DrrTable<4, 4> kDrr4x4;
const DrrTable<4, 1> kDrr4x1;

// One wave per tile (64 threads per work item). Large messages: 256-thread
// workgroups, at most 2 per CU (a narrow HBM access window measured best on
// MI355X); decode-size messages: one tile per wave over every CU.
LaunchPolicy policy_quant() { return {256u, 256u, 2u}; }
LaunchPolicy policy_drr() { return {64u, 256u, 2u}; }

// Below this many large-variant wave tiles per CU a message counts as
// decode-size and takes the narrow variant.
constexpr size_t kSmallTilesPerCu = 8;

}  // namespace

hipError_t launch_quant(const QuantArgs& a, int src_dtype, int fmt, int block, hipStream_t s)
{
    const int lb = __builtin_ctz((unsigned)block) - 5;
    const size_t vec_elems = src_dtype == 0 ? 4 : 8;
    const size_t cus = (size_t)device_cu_count();
    const size_t large_tiles = (a.count + 4 * 64 * vec_elems - 1) / (4 * 64 * vec_elems) * (size_t)a.nsrc;
    const bool small = large_tiles < kSmallTilesPerCu * cus;
    // loads per tile of the chosen variant
    size_t lanes_per_block = (size_t)block / vec_elems;
    size_t u = small ? (lanes_per_block <= 64 ? 1 : lanes_per_block / 64) : 4;
    const size_t tile_elems = u * 64 * vec_elems;
    const size_t tiles = (a.count + tile_elems - 1) / tile_elems * (size_t)a.nsrc;
    dim3 grid, blk;
    launch_geometry(tiles * kWave, small, policy_quant(), grid, blk);
    QuantArgs arg = a;
    void* params[] = {&arg};
    QuantFn fn = small ? kQuantSmall.fn[src_dtype][fmt][lb] : kQuantLarge.fn[src_dtype][fmt][lb];
    return hipLaunchKernel((const void*)fn, grid, blk, params, 0, s);
}

hipError_t launch_drr(const DrrArgs& a, int nsrc, int fmt, bool requant, hipStream_t s)
{
    const size_t cus = (size_t)device_cu_count();
    const size_t len = a.hi - a.lo;
    const bool small = (len + 1023) / 1024 < kSmallTilesPerCu * cus / 2;
    const bool fp32_out = a.out_hp != nullptr && !a.hp_bf16;
    // chunk layout (codes per lane per chunk, chunks per lane); block / CPC <= 64
    int cpc = 16, u = 1;
    if (small) {
        if (a.block <= 256) cpc = 4;
    } else if (fp32_out) {
        if (a.block <= 256) { cpc = 4; u = 4; }
    } else if (a.block <= 512) {
        cpc = 8;
        u = 2;
    }
    const size_t tile = (size_t)kWave * cpc * u;
    const size_t tiles = (len + tile - 1) / tile;
    dim3 grid, blk;
    launch_geometry(tiles * kWave, small, policy_drr(), grid, blk);
    DrrArgs arg = a;
    void* params[] = {&arg};
    const int r = requant ? (a.nout > 1 ? 2 : 1) : 0;
    const DrrFn fn = cpc == 4 ? (u == 4 ? kDrr4x4.fn[fmt][r][nsrc - 1] : kDrr4x1.fn[fmt][r][nsrc - 1])
                   : cpc == 8 ? kDrr8x2.fn[fmt][r][nsrc - 1] : kDrr16x1.fn[fmt][r][nsrc - 1];
    return hipLaunchKernel((const void*)fn, grid, blk, params, 0, s);
}

}  // namespace rx
