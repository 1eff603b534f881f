// drr.hpp -- the fused dequantize -> FP32 sum -> requantize kernel of the
// low-precision collectives on gfx950 (RCCLX article, code-journey.com,
// "Core feature 2: Low-Precision Collectives": FP8 on the wire, "Compute
// precision" FP32). One kernel template serves rx_dequant_reduce_requant
// (one destination) and rx_lp_reduce_scatter_chunk_bcast (the requantized
// chunk pushed to every destination). Each lane layout is instantiated in a
// translation unit of its own (drr_<CPC>x<U>.hip) so the build compiles them
// in parallel.
#pragma once

#include <array>
#include <utility>

#include "rx_device.hpp"
#include "rx_internal.hpp"

namespace rx {

using DrrFn = void (*)(DrrArgs);

// [fmt][mode][nsrc - 1]; modes: 0 sum, 1 requant, 2 requant with the codes
// pushed to every destination, 3 requant with the dequantized result written
// to every rank's buffer
enum { kDrrSum = 0, kDrrRequant = 1, kDrrRequantPush = 2, kDrrRequantAll = 3 };
struct DrrFns {
    DrrFn fn[2][4][kMaxSrc];
};

const DrrFns& drr_fns_16x1();
const DrrFns& drr_fns_8x2();
const DrrFns& drr_fns_4x4();
const DrrFns& drr_fns_4x1();
// Staged 16 x 1 kernels for whole tiles, [hp_bf16]
const DrrFns& drr_fns_16x1_staged(int hp_bf16);
// Whole-tile kernels (k_drr_whole), 16 x 1
const DrrFns& drr_fns_16x1_whole();
// Decode-size kernels for ranges of whole tiles (k_drr_tile1), 4 x 1
const DrrFns& drr_fns_4x1_tile1();
// Prefetching whole-tile kernels (k_drr_pf): codes only (one destination)
// in 16 x 1, [fmt][nsrc - 1]; the one-source dequantization (SUM) in 4 x 4
// and 8 x 2, [fmt]; the staged requantization with a high-precision output
// (k_drr_staged_pf), [hp_bf16][fmt][nsrc - 1]
struct DrrPfFns {
    DrrFn codes16[2][kMaxSrc];
    DrrFn sum44[2];
    DrrFn sum82[2];
    DrrFn staged[2][2][kMaxSrc];
};
const DrrPfFns& drr_fns_pf();

namespace drr_detail {


// Lane layout of a wave tile of 64 * CPC * U codes: lane l owns U chunks of
// CPC consecutive codes, chunk u at tile offset (u * 64 + l) * CPC. Every
// load and store instruction then covers one contiguous run (64 lanes x CPC
// codes, or their 2- or 4-byte outputs). Layouts used:
//   CPC 16, U 1: dwordx4 code loads (any block size); code-only output, and
//                (k_drr_staged) FP32 or BF16 output from several sources with
//                the output staged through LDS into contiguous stores;
//   CPC  8, U 2: BF16 output from one source, 16-byte stores contiguous
//                across the wave;
//   CPC  4, U 4: FP32 output from one source, 16-byte stores contiguous
//                across the wave;
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
    } else {
        // codes [e, count) byte by byte, the rest code 0 (decodes to +0):
        // each byte loaded from an index clamped to count - 1 (in bounds,
        // count >= 1) and masked afterwards, so the loads carry no branches
        // and are all in flight before the first use
        uint32_t b[CPC];
#pragma unroll
        for (int k = 0; k < CPC; ++k)
            b[k] = p[e + k < count ? e + k : count - 1];
#pragma unroll
        for (int q = 0; q < CPC / 4; ++q) x.w[q] = 0u;
#pragma unroll
        for (int k = 0; k < CPC; ++k)
            x.w[k / 4] |= (e + k < count ? b[k] : 0u) << (8 * (k & 3));
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

// One block scale. The decode-size layout (CPC 4, U 1, only launched for
// decode-size messages) stores them nontemporal: the scattered 4-byte stores
// then leave no partly written lines for the end-of-kernel cache write-back
// (measured 6-7% faster there); the large layouts keep them in L2, where the
// lines fill up before they are written back (nontemporal: up to 19% slower).
// A compile-time choice: a run-time branch between the two stores is merged
// into one plain store by the compiler.
template <bool NT>
__device__ __forceinline__ void store_scale(float* p, float s)
{
    if constexpr (NT)
        __builtin_nontemporal_store(s, p);
    else
        *p = s;
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

// High-precision output of a whole 16 x 1 tile staged through LDS: lane l's
// 16 values, as SL = 4 (FP32) or 2 (BF16) 16-byte slots, become row l of the
// wave's stage (rows of SL + 1 slots, one of them padding against bank
// conflicts); store instruction u then takes slot u * 64 + l of the tile --
// row u * 64 / SL + l / SL, slot l % SL -- so each of the tile's SL stores
// writes one contiguous 1 KiB run (nontemporal), where the unstaged 16 x 1
// layout writes strided 16-byte pieces. The stage belongs to one wave; the
// waits keep the previous tile's reads before this tile's writes and the
// writes before the reads.
constexpr int kStageSlots = 64 * 5;

__device__ __forceinline__ void stage_wait()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
}

template <bool BF16>
__device__ __forceinline__ void stage_hp(u32x4* stage, int lane, const float* h, u32x4* piece)
{
    constexpr int SL = BF16 ? 2 : 4;
    stage_wait();
#pragma unroll
    for (int q = 0; q < SL; ++q) {
        u32x4 v;
        if constexpr (BF16) {
#pragma unroll
            for (int k = 0; k < 4; ++k) v[k] = pack_bf16(h[8 * q + 2 * k], h[8 * q + 2 * k + 1]);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) v[k] = __builtin_bit_cast(uint32_t, h[4 * q + k]);
        }
        stage[lane * (SL + 1) + q] = v;
    }
    stage_wait();
#pragma unroll
    for (int u = 0; u < SL; ++u)
        piece[u] = stage[(u * (kWave / SL) + lane / SL) * (SL + 1) + lane % SL];
}

// The SL staged pieces into one output, whose tile starts at 16-byte vector
// v0 (FP32: 4 per 16 codes, BF16: 2).
template <bool BF16>
__device__ __forceinline__ void store_staged(void* out, size_t v0, int lane, const u32x4* piece)
{
    constexpr int SL = BF16 ? 2 : 4;
#pragma unroll
    for (int u = 0; u < SL; ++u)
        st16_stream(out, v0 + (size_t)u * kWave + lane, piece[u]);
}

// Stage a whole tile's output once and write it to NOUT outputs.
template <int NOUT, bool BF16>
__device__ __forceinline__ void staged_out(void* const* outs, size_t c_tile, u32x4* stage, int lane,
                                           const float* h)
{
    u32x4 piece[4];
    stage_hp<BF16>(stage, lane, h, piece);
#pragma unroll
    for (int j = 0; j < NOUT; ++j)
        store_staged<BF16>(outs[j], c_tile * (BF16 ? 2 : 4), lane, piece);
}

// OUT (requantization only): kDrrRequant -> out_codes[0] / out_scales[0]
// (+ out_hp); kDrrRequantPush -> the codes and scales to N destinations, one
// per rank (the low-precision tree step's push); kDrrRequantAll -> only the
// dequantized result, into N buffers out_hps[j] (every rank's final values
// in a one-device allreduce).
// The arithmetic and stores of one wave tile whose codes and scales are in
// registers (x, sc: chunk u of source r; c, e, b: this lane's chunk index,
// first code and block of chunk u; whole / valid: chunk u lies wholly /
// partly inside the range): dequantize, sum in source order, then store the
// sum (SUM) or requantize and store as OUT says.
template <int F, int N, bool REQUANT, int CPC, int U, int OUT>
__device__ __forceinline__ void drr_finish(const DrrArgs& a, const Chunk<CPC> (&x)[N][U], const float (&sc)[N][U],
                                           const size_t (&c)[U], const size_t (&e)[U], const size_t (&b)[U],
                                           const bool (&whole)[U], const bool (&valid)[U], size_t count, int lane,
                                           int lpb)
{
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
        if constexpr (OUT == kDrrRequantPush) {
            // push the chunk to every destination (one per rank: nout == N,
            // so the loop unrolls and the pointers load once)
#pragma unroll
            for (int j = 0; j < N; ++j)
                store_codes<CPC>(static_cast<uint8_t*>(a.out_codes[j]), c[u], e[u], count, whole[u], q);
            if (valid[u] && (lane & (lpb - 1)) == 0) {
#pragma unroll
                for (int j = 0; j < N; ++j)
                    store_scale<CPC == 4 && U == 1>(a.out_scales[j] + b[u], s2);
            }
        } else if constexpr (OUT == kDrrRequant) {
            store_codes<CPC>(static_cast<uint8_t*>(a.out_codes[0]), c[u], e[u], count, whole[u], q);
            if (valid[u] && (lane & (lpb - 1)) == 0)
                store_scale<CPC == 4 && U == 1>(a.out_scales[0] + b[u], s2);
        }

        if constexpr (OUT == kDrrRequantAll) {
            float h[CPC];
            dequant<F, CPC>(q, s2, h);
#pragma unroll
            for (int j = 0; j < N; ++j)
                store_hp<CPC>(a.out_hps[j], a.hp_bf16 != 0, c[u], e[u], count, whole[u], h);
        } else if (a.out_hp) {
            float h[CPC];
            dequant<F, CPC>(q, s2, h);
            store_hp<CPC>(a.out_hp, a.hp_bf16 != 0, c[u], e[u], count, whole[u], h);
        }
    }
}

// One wave tile of k_drr. WHOLE: every chunk of the tile lies inside the
// range (all tiles but a ragged last one); that instance has no per-lane
// bounds branches around its loads and stores.
template <int F, int N, bool REQUANT, int CPC, int U, int OUT, bool WHOLE>
__device__ __forceinline__ void drr_tile(const DrrArgs& a, uint32_t t, int lane, size_t c0,
                                         size_t count, int bshift, int lpb)
{
    size_t c[U], e[U], b[U];
    bool whole[U], valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        c[u] = c0 + ((size_t)t * U + u) * kWave + lane;  // this lane's chunk u
        e[u] = c[u] * CPC;
        whole[u] = WHOLE || e[u] + CPC <= count;
        valid[u] = WHOLE || e[u] < count;
        b[u] = e[u] >> bshift;
    }

    Chunk<CPC> x[N][U];
    float sc[N][U];
#pragma unroll
    for (int r = 0; r < N; ++r) {
        const uint8_t* cp = static_cast<const uint8_t*>(a.codes[r]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (WHOLE || CPC * U == 4) {
                // whole tiles; and the decode-size layout's partial tile, byte
                // by byte in every lane (4 loads per source, no branches, one
                // wait for all sources)
                x[r][u] = load_chunk<CPC>(cp, c[u], e[u], count, WHOLE);
            } else {
                // a large layout's partial tile: whole chunks load as vectors
                // and only the chunk that straddles the end byte by byte
                // (byte loads in every lane would hold CPC x U x N registers
                // for the whole kernel)
                if (whole[u])
                    x[r][u] = load_chunk<CPC>(cp, c[u], e[u], count, true);
                else if (valid[u])
                    x[r][u] = load_chunk<CPC>(cp, c[u], e[u], count, false);
                else {
#pragma unroll
                    for (int q = 0; q < CPC / 4; ++q) x[r][u].w[q] = 0u;
                }
            }
            sc[r][u] = valid[u] ? a.scales[r][b[u]] : 0.0f;
        }
    }
    drr_finish<F, N, REQUANT, CPC, U, OUT>(a, x, sc, c, e, b, whole, valid, count, lane, lpb);
}

template <int F, int N, bool REQUANT, int CPC, int U, int OUT>
__global__ __launch_bounds__(256) void k_drr(DrrArgs a)
{
    const int lane = lane_id();
    const uint32_t wave_in_wg = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t waves_per_wg = blockDim.x / kWave;
    const size_t count = a.hi;                                    // end of the range
    constexpr size_t kTile = (size_t)kWave * CPC * U;             // codes per wave tile
    const uint32_t ntiles = (uint32_t)((a.hi - a.lo + kTile - 1) / kTile);
    uint32_t wave, step;
    if (a.xcd_ranges > 1) {
        // one tile per 64-thread workgroup; XCD x takes tiles [x R, x R + R)
        // (R = xcd_ranges, a whole number of 128-byte lines of block scales,
        // so no XCD leaves a line of scales partly written); workgroups past
        // the last tile do nothing
        wave = (blockIdx.x % kXcds) * (uint32_t)a.xcd_ranges + blockIdx.x / kXcds;
        step = ntiles;
    } else {
        const uint32_t wg = a.xcd_ranges ? xcd_contiguous(blockIdx.x, gridDim.x) : blockIdx.x;
        wave = wg * waves_per_wg + wave_in_wg;
        step = gridDim.x * waves_per_wg;
    }
    const size_t c0 = a.lo / CPC;                                 // lo is a block multiple
    const int lpb = a.block / CPC;                                // lanes per block: <= 64
    const int bshift = __builtin_ctz((unsigned)a.block);

    for (uint32_t t = wave; t < ntiles; t += step) {
        if (a.lo + ((size_t)t + 1) * kTile <= count)
            drr_tile<F, N, REQUANT, CPC, U, OUT, true>(a, t, lane, c0, count, bshift, lpb);
        else
            drr_tile<F, N, REQUANT, CPC, U, OUT, false>(a, t, lane, c0, count, bshift, lpb);
    }
}

// True if a source's code or scale pointer is null (never, for a validated
// call). A kernel that adds it to its exit test has every source pointer
// loaded before that branch, together with the range, instead of after it:
// one scalar round trip before the first code load instead of two. Written
// as a minimum over the pointers (two scalar instructions each).
template <int N>
__device__ __forceinline__ bool any_source_null(const DrrArgs& a)
{
    uint32_t m = ~0u;
#pragma unroll
    for (int r = 0; r < N; ++r) {
        const uint32_t c = ptr_nonzero(a.codes[r]), s = ptr_nonzero(a.scales[r]);
        m = m < c ? m : c;
        m = m < s ? m : s;
    }
    return m == 0;
}

// Decode-size ranges of whole tiles, every mode: one tile per 64-thread
// workgroup, XCD x taking tiles [x R, x R + R) (R = xcd_ranges, whole lines
// of block scales), without k_drr's loop and partial-tile path, and with
// the source pointers in the exit test (their loads go out with the
// range's). Against k_drr: the LP tree step's push of a 32K-code chunk
// 2.54 -> 2.41 us, the requantization of 8 x 256K codes into one
// destination with the BF16 output 2.73 -> 2.66 us, the one-source
// dequantization 2.02 -> 1.97 us; the 8-source flat LP sum 2.33 -> 2.34.
template <int F, int N, bool REQUANT, int CPC, int U, int OUT>
__global__ __launch_bounds__(256) void k_drr_tile1(DrrArgs a)
{
    constexpr size_t kTile = (size_t)kWave * CPC * U;
    const uint32_t ntiles = (uint32_t)((a.hi - a.lo) / kTile);
    const uint32_t t = (blockIdx.x % kXcds) * (uint32_t)a.xcd_ranges + blockIdx.x / kXcds;
    if ((t >= ntiles) | any_source_null<N>(a))
        return;
    drr_tile<F, N, REQUANT, CPC, U, OUT, true>(a, t, lane_id(), a.lo / CPC, a.hi, __builtin_ctz((unsigned)a.block),
                                               a.block / CPC);
}

// Large messages, whole tiles only: tiles [0, hi / (64 CPC U)) of a range
// that starts at code 0 (the launcher offsets every pointer to the start of
// the range and runs k_drr over the ragged remainder). Without k_drr's
// choice between the whole-tile and the partial-tile path inside the loop,
// codes only, 8 x 16M codes E4M3/128: 27.2 -> 26.3 us (8 x 64M E5M2/256:
// 102.3 -> 100.4 us).
template <int F, int N, bool REQUANT, int CPC, int U, int OUT>
__global__ __launch_bounds__(256) void k_drr_whole(DrrArgs a)
{
    const int lane = lane_id();
    const uint32_t wave_in_wg = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t waves_per_wg = blockDim.x / kWave;
    constexpr size_t kTile = (size_t)kWave * CPC * U;
    const uint32_t ntiles = (uint32_t)(a.hi / kTile);
    const uint32_t wg = a.xcd_ranges ? xcd_contiguous(blockIdx.x, gridDim.x) : blockIdx.x;
    const uint32_t wave = wg * waves_per_wg + wave_in_wg;
    const uint32_t step = gridDim.x * waves_per_wg;
    const int lpb = a.block / CPC;
    const int bshift = __builtin_ctz((unsigned)a.block);
    for (uint32_t t = wave; t < ntiles; t += step)
        drr_tile<F, N, REQUANT, CPC, U, OUT, true>(a, t, lane, 0, a.hi, bshift, lpb);
}

// Codes and scales of whole tile t (every chunk inside the range) into
// registers.
template <int N, int CPC, int U>
__device__ __forceinline__ void drr_load_whole(Chunk<CPC> (&x)[N][U], float (&sc)[N][U], const DrrArgs& a, uint32_t t,
                                               int lane, int bshift)
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const size_t c = ((size_t)t * U + u) * kWave + lane;
        const size_t e = c * CPC;
#pragma unroll
        for (int r = 0; r < N; ++r) {
            x[r][u] = load_chunk<CPC>(static_cast<const uint8_t*>(a.codes[r]), c, e, a.hi, true);
            sc[r][u] = a.scales[r][e >> bshift];
        }
    }
}

template <int F, int N, bool REQUANT, int CPC, int U, int OUT>
__device__ __forceinline__ void drr_finish_whole(const Chunk<CPC> (&x)[N][U], const float (&sc)[N][U],
                                                 const DrrArgs& a, uint32_t t, int lane, int bshift, int lpb)
{
    size_t c[U], e[U], b[U];
    bool yes[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        c[u] = ((size_t)t * U + u) * kWave + lane;
        e[u] = c[u] * CPC;
        b[u] = e[u] >> bshift;
        yes[u] = true;
    }
    drr_finish<F, N, REQUANT, CPC, U, OUT>(a, x, sc, c, e, b, yes, yes, a.hi, lane, lpb);
}

// k_drr_whole with the next tile's codes and scales loaded into a second
// register buffer before the current tile's arithmetic (the two buffers in
// turn and the wave's last tile peeled off, so that no register copy crosses
// the loop and every prefetch in it is unconditional). With one or two
// workgroups per CU a wave's arithmetic otherwise leaves its loads idle:
// codes only, 8 x 256M codes E5M2/256: 441.8 -> 425.4 us (one workgroup per
// CU); one source to FP32, 16M codes E4M3/128: 16.36 -> 15.66 us; to BF16,
// 64M codes E5M2/256: 36.2 -> 35.0 us (two per CU).
template <int F, int N, bool REQUANT, int CPC, int U, int OUT>
__global__ __launch_bounds__(256) void k_drr_pf(DrrArgs a)
{
    const int lane = lane_id();
    const uint32_t wave_in_wg = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t waves_per_wg = blockDim.x / kWave;
    constexpr size_t kTile = (size_t)kWave * CPC * U;
    const uint32_t ntiles = (uint32_t)(a.hi / kTile);
    const uint32_t wg = a.xcd_ranges ? xcd_contiguous(blockIdx.x, gridDim.x) : blockIdx.x;
    uint32_t t = wg * waves_per_wg + wave_in_wg;
    const uint32_t step = gridDim.x * waves_per_wg;
    const int lpb = a.block / CPC;
    const int bshift = __builtin_ctz((unsigned)a.block);
    if (t >= ntiles)
        return;
    Chunk<CPC> xa[N][U], xb[N][U];
    float sa[N][U], sb[N][U];
    uint32_t n = (ntiles - t + step - 1) / step;   // tiles of this wave, >= 1
    drr_load_whole<N, CPC, U>(xa, sa, a, t, lane, bshift);
    for (;;) {
        if (n == 1) {
            drr_finish_whole<F, N, REQUANT, CPC, U, OUT>(xa, sa, a, t, lane, bshift, lpb);
            break;
        }
        drr_load_whole<N, CPC, U>(xb, sb, a, t + step, lane, bshift);
        drr_finish_whole<F, N, REQUANT, CPC, U, OUT>(xa, sa, a, t, lane, bshift, lpb);
        t += step;
        --n;
        if (n == 1) {
            drr_finish_whole<F, N, REQUANT, CPC, U, OUT>(xb, sb, a, t, lane, bshift, lpb);
            break;
        }
        drr_load_whole<N, CPC, U>(xa, sa, a, t + step, lane, bshift);
        drr_finish_whole<F, N, REQUANT, CPC, U, OUT>(xb, sb, a, t, lane, bshift, lpb);
        t += step;
        --n;
    }
}

// The 16 x 1 layout with the high-precision output (FP32, or BF16 when
// BF16) staged through LDS, for whole tiles of 1024 codes only: tiles
// [0, hi / 1024); the launcher passes every pointer already offset to the
// start of the range (lo == 0 here) and runs the unstaged kernel over a
// ragged remainder. Lane l owns chunk l of 16 codes (one 16-byte load per
// source); sums, requantization and code / scale stores as in drr_tile.
// Launched only for modes with a high-precision output (out_hp, or out_hps
// for kDrrRequantAll). The range offset and an out_hp check, both removed
// here, made the compiler schedule the loop 4% slower (8 x 64M codes
// E5M2/256 with BF16 output: 127.3 against 121.7 us).
// The staged kernel's tile t in two parts: its codes and scales into
// registers, then the sums, requantization and stores (the output through
// the wave's LDS stage).
template <int N>
__device__ __forceinline__ void drr_staged_load(Chunk<16> (&x)[N], float (&sc)[N], const DrrArgs& a, uint32_t t,
                                                int lane, int bshift)
{
    const size_t c = (size_t)t * kWave + lane;
    const size_t e = c * 16;
#pragma unroll
    for (int r = 0; r < N; ++r) {
        x[r] = load_chunk<16>(static_cast<const uint8_t*>(a.codes[r]), c, e, a.hi, true);
        sc[r] = a.scales[r][e >> bshift];
    }
}

template <int F, int N, bool REQUANT, int OUT, bool BF16>
__device__ __forceinline__ void drr_staged_finish(const Chunk<16> (&x)[N], const float (&sc)[N], const DrrArgs& a,
                                                  uint32_t t, int lane, int lpb, int bshift, u32x4* stage)
{
    const size_t c_tile = (size_t)t * kWave;
    const size_t c = c_tile + lane;
    const size_t e = c * 16;
    const size_t b = e >> bshift;
    float S[16];
    dequant<F, 16>(x[0].w, sc[0], S);
#pragma unroll
    for (int r = 1; r < N; ++r) {
        float d[16];
        dequant<F, 16>(x[r].w, sc[r], d);
#pragma unroll
        for (int k = 0; k < 16; ++k)
            S[k] = S[k] + d[k];
    }
    if constexpr (!REQUANT) {
        staged_out<1, BF16>(&a.out_hp, c_tile, stage, lane, S);
        return;
    }
    float m = __builtin_fabsf(S[0]);
#pragma unroll
    for (int k = 1; k < 16; ++k)
        m = __builtin_fmaxf(m, __builtin_fabsf(S[k]));
    const float A = bits_f32(group_max_rt(__builtin_bit_cast(uint32_t, m), lpb));
    float s2, r2;
    block_scale<F>(A, s2, r2);
    uint32_t q[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
        q[p] = f32x4_to_fp8<F>(clamp_fmax<F>(S[4 * p + 0] * r2), clamp_fmax<F>(S[4 * p + 1] * r2),
                               clamp_fmax<F>(S[4 * p + 2] * r2), clamp_fmax<F>(S[4 * p + 3] * r2));
    if constexpr (OUT == kDrrRequantPush) {
#pragma unroll
        for (int j = 0; j < N; ++j)
            store_codes<16>(static_cast<uint8_t*>(a.out_codes[j]), c, e, a.hi, true, q);
        if ((lane & (lpb - 1)) == 0) {
#pragma unroll
            for (int j = 0; j < N; ++j)
                store_scale<false>(a.out_scales[j] + b, s2);
        }
    } else if constexpr (OUT == kDrrRequant) {
        store_codes<16>(static_cast<uint8_t*>(a.out_codes[0]), c, e, a.hi, true, q);
        if ((lane & (lpb - 1)) == 0)
            store_scale<false>(a.out_scales[0] + b, s2);
    }
    float h[16];
    dequant<F, 16>(q, s2, h);
    if constexpr (OUT == kDrrRequantAll)
        staged_out<N, BF16>(a.out_hps, c_tile, stage, lane, h);
    else
        staged_out<1, BF16>(&a.out_hp, c_tile, stage, lane, h);
}

template <int F, int N, bool REQUANT, int OUT, bool BF16>
__global__ __launch_bounds__(256) void k_drr_staged(DrrArgs a)
{
    __shared__ u32x4 stage_mem[256 / kWave][kStageSlots];   // one region per wave
    const int lane = lane_id();
    const uint32_t wave_in_wg = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t wg = a.xcd_ranges ? xcd_contiguous(blockIdx.x, gridDim.x) : blockIdx.x;
    const uint32_t wave = wg * (blockDim.x / kWave) + wave_in_wg;
    const uint32_t step = gridDim.x * (blockDim.x / kWave);
    const uint32_t ntiles = (uint32_t)(a.hi / ((size_t)kWave * 16));
    const int lpb = a.block / 16;                                 // lanes per block: <= 64
    const int bshift = __builtin_ctz((unsigned)a.block);
    u32x4* stage = stage_mem[wave_in_wg];

    for (uint32_t t = wave; t < ntiles; t += step) {
        Chunk<16> x[N];
        float sc[N];
        drr_staged_load<N>(x, sc, a, t, lane, bshift);
        drr_staged_finish<F, N, REQUANT, OUT, BF16>(x, sc, a, t, lane, lpb, bshift, stage);
    }
}

// k_drr_staged with the next tile's codes and scales loaded into a second
// register buffer before the current tile's arithmetic (as k_drr_pf):
// requantization with the output staged, from 256 tiles per CU at one
// workgroup per CU (8 x 256M codes E5M2/256 with BF16 output: 500.4 ->
// 478.1 us; 8 x 64M: 120.3 -> 119.3 us; at 8 x 16M codes with FP32 output,
// 64 tiles per CU, 1.7% slower).
template <int F, int N, bool REQUANT, int OUT, bool BF16>
__global__ __launch_bounds__(256) void k_drr_staged_pf(DrrArgs a)
{
    __shared__ u32x4 stage_mem[256 / kWave][kStageSlots];   // one region per wave
    const int lane = lane_id();
    const uint32_t wave_in_wg = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t wg = a.xcd_ranges ? xcd_contiguous(blockIdx.x, gridDim.x) : blockIdx.x;
    uint32_t t = wg * (blockDim.x / kWave) + wave_in_wg;
    const uint32_t step = gridDim.x * (blockDim.x / kWave);
    const uint32_t ntiles = (uint32_t)(a.hi / ((size_t)kWave * 16));
    const int lpb = a.block / 16;
    const int bshift = __builtin_ctz((unsigned)a.block);
    u32x4* stage = stage_mem[wave_in_wg];
    if (t >= ntiles)
        return;
    Chunk<16> xa[N], xb[N];
    float sa[N], sb[N];
    uint32_t n = (ntiles - t + step - 1) / step;   // tiles of this wave, >= 1
    drr_staged_load<N>(xa, sa, a, t, lane, bshift);
    for (;;) {
        if (n == 1) {
            drr_staged_finish<F, N, REQUANT, OUT, BF16>(xa, sa, a, t, lane, lpb, bshift, stage);
            break;
        }
        drr_staged_load<N>(xb, sb, a, t + step, lane, bshift);
        drr_staged_finish<F, N, REQUANT, OUT, BF16>(xa, sa, a, t, lane, lpb, bshift, stage);
        t += step;
        --n;
        if (n == 1) {
            drr_staged_finish<F, N, REQUANT, OUT, BF16>(xb, sb, a, t, lane, lpb, bshift, stage);
            break;
        }
        drr_staged_load<N>(xa, sa, a, t + step, lane, bshift);
        drr_staged_finish<F, N, REQUANT, OUT, BF16>(xb, sb, a, t, lane, lpb, bshift, stage);
        t += step;
        --n;
    }
}


template <int F, bool R, int CPC, int U, int OUT, int... I>
void fill_row(DrrFn* row, std::integer_sequence<int, I...>)
{
    ((row[I] = &k_drr<F, I + 1, R, CPC, U, OUT>), ...);
}

template <int CPC, int U>
DrrFns make_fns()
{
    DrrFns t{};
    const auto seq = std::make_integer_sequence<int, kMaxSrc>{};
    fill_row<0, false, CPC, U, kDrrSum>(t.fn[0][kDrrSum], seq);
    fill_row<0, true, CPC, U, kDrrRequant>(t.fn[0][kDrrRequant], seq);
    fill_row<0, true, CPC, U, kDrrRequantPush>(t.fn[0][kDrrRequantPush], seq);
    fill_row<0, true, CPC, U, kDrrRequantAll>(t.fn[0][kDrrRequantAll], seq);
    fill_row<1, false, CPC, U, kDrrSum>(t.fn[1][kDrrSum], seq);
    fill_row<1, true, CPC, U, kDrrRequant>(t.fn[1][kDrrRequant], seq);
    fill_row<1, true, CPC, U, kDrrRequantPush>(t.fn[1][kDrrRequantPush], seq);
    fill_row<1, true, CPC, U, kDrrRequantAll>(t.fn[1][kDrrRequantAll], seq);
    return t;
}

template <int F, bool R, int CPC, int U, int OUT, int... I>
void fill_whole_row(DrrFn* row, std::integer_sequence<int, I...>)
{
    ((row[I] = &k_drr_whole<F, I + 1, R, CPC, U, OUT>), ...);
}

template <int F, bool R, int CPC, int U, int OUT, int... I>
void fill_tile1_row(DrrFn* row, std::integer_sequence<int, I...>)
{
    ((row[I] = &k_drr_tile1<F, I + 1, R, CPC, U, OUT>), ...);
}

// every mode
template <int CPC, int U>
DrrFns make_tile1_fns()
{
    DrrFns t{};
    const auto seq = std::make_integer_sequence<int, kMaxSrc>{};
    fill_tile1_row<0, false, CPC, U, kDrrSum>(t.fn[0][kDrrSum], seq);
    fill_tile1_row<0, true, CPC, U, kDrrRequant>(t.fn[0][kDrrRequant], seq);
    fill_tile1_row<0, true, CPC, U, kDrrRequantPush>(t.fn[0][kDrrRequantPush], seq);
    fill_tile1_row<0, true, CPC, U, kDrrRequantAll>(t.fn[0][kDrrRequantAll], seq);
    fill_tile1_row<1, false, CPC, U, kDrrSum>(t.fn[1][kDrrSum], seq);
    fill_tile1_row<1, true, CPC, U, kDrrRequant>(t.fn[1][kDrrRequant], seq);
    fill_tile1_row<1, true, CPC, U, kDrrRequantPush>(t.fn[1][kDrrRequantPush], seq);
    fill_tile1_row<1, true, CPC, U, kDrrRequantAll>(t.fn[1][kDrrRequantAll], seq);
    return t;
}

template <int CPC, int U>
DrrFns make_whole_fns()
{
    DrrFns t{};
    const auto seq = std::make_integer_sequence<int, kMaxSrc>{};
    fill_whole_row<0, false, CPC, U, kDrrSum>(t.fn[0][kDrrSum], seq);
    fill_whole_row<0, true, CPC, U, kDrrRequant>(t.fn[0][kDrrRequant], seq);
    fill_whole_row<0, true, CPC, U, kDrrRequantPush>(t.fn[0][kDrrRequantPush], seq);
    fill_whole_row<0, true, CPC, U, kDrrRequantAll>(t.fn[0][kDrrRequantAll], seq);
    fill_whole_row<1, false, CPC, U, kDrrSum>(t.fn[1][kDrrSum], seq);
    fill_whole_row<1, true, CPC, U, kDrrRequant>(t.fn[1][kDrrRequant], seq);
    fill_whole_row<1, true, CPC, U, kDrrRequantPush>(t.fn[1][kDrrRequantPush], seq);
    fill_whole_row<1, true, CPC, U, kDrrRequantAll>(t.fn[1][kDrrRequantAll], seq);
    return t;
}

template <int F, int... I>
void fill_pf_codes_row(DrrFn* row, std::integer_sequence<int, I...>)
{
    ((row[I] = &k_drr_pf<F, I + 1, true, 16, 1, kDrrRequant>), ...);
}

template <int F, bool BF16, int... I>
void fill_pf_staged_row(DrrFn* row, std::integer_sequence<int, I...>)
{
    ((row[I] = &k_drr_staged_pf<F, I + 1, true, kDrrRequant, BF16>), ...);
}

inline DrrPfFns make_pf_fns()
{
    DrrPfFns t{};
    const auto seq = std::make_integer_sequence<int, kMaxSrc>{};
    fill_pf_codes_row<0>(t.codes16[0], seq);
    fill_pf_codes_row<1>(t.codes16[1], seq);
    fill_pf_staged_row<0, false>(t.staged[0][0], seq);
    fill_pf_staged_row<1, false>(t.staged[0][1], seq);
    fill_pf_staged_row<0, true>(t.staged[1][0], seq);
    fill_pf_staged_row<1, true>(t.staged[1][1], seq);
    t.sum44[0] = &k_drr_pf<0, 1, false, 4, 4, kDrrSum>;
    t.sum44[1] = &k_drr_pf<1, 1, false, 4, 4, kDrrSum>;
    t.sum82[0] = &k_drr_pf<0, 1, false, 8, 2, kDrrSum>;
    t.sum82[1] = &k_drr_pf<1, 1, false, 8, 2, kDrrSum>;
    return t;
}

template <int F, bool R, int OUT, bool BF16, int... I>
void fill_staged_row(DrrFn* row, std::integer_sequence<int, I...>)
{
    ((row[I] = &k_drr_staged<F, I + 1, R, OUT, BF16>), ...);
}

template <bool BF16>
DrrFns make_staged_fns()
{
    DrrFns t{};
    const auto seq = std::make_integer_sequence<int, kMaxSrc>{};
    fill_staged_row<0, false, kDrrSum, BF16>(t.fn[0][kDrrSum], seq);
    fill_staged_row<0, true, kDrrRequant, BF16>(t.fn[0][kDrrRequant], seq);
    fill_staged_row<0, true, kDrrRequantPush, BF16>(t.fn[0][kDrrRequantPush], seq);
    fill_staged_row<0, true, kDrrRequantAll, BF16>(t.fn[0][kDrrRequantAll], seq);
    fill_staged_row<1, false, kDrrSum, BF16>(t.fn[1][kDrrSum], seq);
    fill_staged_row<1, true, kDrrRequant, BF16>(t.fn[1][kDrrRequant], seq);
    fill_staged_row<1, true, kDrrRequantPush, BF16>(t.fn[1][kDrrRequantPush], seq);
    fill_staged_row<1, true, kDrrRequantAll, BF16>(t.fn[1][kDrrRequantAll], seq);
    return t;
}

}  // namespace drr_detail
}  // namespace rx
