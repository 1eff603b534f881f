// ceiling.hip -- plain streaming kernels (read, write, copy; 16 bytes per
// lane per access) that measure the HBM ceilings the hot-path kernels are
// compared against on the same GPU in the same run.
#include <array>
#include <stdint.h>
#include <stdio.h>
#include <utility>

#include "rx_device.hpp"
#include "rx_internal.hpp"
#include "rx_testhooks.h"

namespace rx {
namespace {

constexpr int kCeilU = 4;                               // vectors per lane per tile
constexpr size_t kCeilTile = (size_t)kWave * kCeilU;    // vectors per wave tile

template <bool NT>
__device__ __forceinline__ u32x4 ld(const void* p, size_t v)
{
    if constexpr (NT) return ld16_stream(p, v);
    else return ld16(p, v);
}

template <bool NT>
__device__ __forceinline__ void st(void* p, size_t v, u32x4 x)
{
    if constexpr (NT) st16_stream(p, v, x);
    else st16(p, v, x);
}

// XOR of a 16-byte value over the 64 lanes of the wave.
__device__ __forceinline__ u32x4 wave_xor(u32x4 v)
{
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            v[q] ^= (uint32_t)__shfl_xor((int)v[q], m, kWave);
    }
    return v;
}

// Wave tiles of kCeilU contiguous 64-vector rows, grid-stride over the waves
// of the launch. KIND 0: read, XOR into a per-wave sum written once at the
// end (16 bytes per wave); 1: write a constant pattern; 2: copy; 3: no
// memory access at all (the launch alone). The loop covers whole tiles only,
// with no bounds checks inside it (checks inside a tile loop serialise the
// loads of a wave); the partial last tile, if any, is done after the loop by
// the wave whose turn it would be.
template <int KIND, bool NT>
__global__ __launch_bounds__(256) void k_stream(const void* __restrict__ src, void* __restrict__ dst,
                                                size_t nvec, u32x4 pattern)
{
    const size_t waves = (size_t)gridDim.x * (blockDim.x / kWave);
    const size_t wave = (size_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const size_t lane = threadIdx.x % kWave;
    u32x4 acc = {0u, 0u, 0u, 0u};
    if constexpr (KIND == 3) return;
    const size_t ntiles = nvec / kCeilTile;
    for (size_t t = wave; t < ntiles; t += waves) {
        const size_t base = t * kCeilTile + lane;
        if constexpr (KIND == 0) {
            u32x4 x[kCeilU];
#pragma unroll
            for (int u = 0; u < kCeilU; ++u) x[u] = ld<NT>(src, base + (size_t)u * kWave);
#pragma unroll
            for (int u = 0; u < kCeilU; ++u) acc ^= x[u];
        } else if constexpr (KIND == 1) {
#pragma unroll
            for (int u = 0; u < kCeilU; ++u) st<NT>(dst, base + (size_t)u * kWave, pattern);
        } else {
            u32x4 x[kCeilU];
#pragma unroll
            for (int u = 0; u < kCeilU; ++u) x[u] = ld<NT>(src, base + (size_t)u * kWave);
#pragma unroll
            for (int u = 0; u < kCeilU; ++u) st<NT>(dst, base + (size_t)u * kWave, x[u]);
        }
    }
    if (ntiles * kCeilTile < nvec && wave == ntiles % waves) {
        for (int u = 0; u < kCeilU; ++u) {
            const size_t v = ntiles * kCeilTile + lane + (size_t)u * kWave;
            if (v >= nvec) break;
            if constexpr (KIND == 0) acc ^= ld16(src, v);
            else if constexpr (KIND == 1) st16(dst, v, pattern);
            else st16(dst, v, ld16(src, v));
        }
    }
    if constexpr (KIND == 0) {
        acc = wave_xor(acc);
        if (lane == 0) st16(dst, wave, acc);
    }
}

// Mixed read/write ceilings: the access patterns of the hot-path kernels
// with their arithmetic replaced by XOR, so their rate is what the memory
// system gives that mix of reads and writes.
//   reduce: NSRC source streams read at the same index, one stream written
//           (NSRC : 1, the flat reduce's pattern; NSRC = 1 is a copy);
//   narrow: one stream read, one written at 1/K of its bytes (16 bytes read
//           and 16/K written per lane: the quantizer's pattern, K = 4 for
//           FP32 and 2 for BF16 input).
// Whole tiles in the loop, the partial last tile after it (as k_stream).
// PF: each wave loads its next tile into a second register buffer before it
// writes the current one; the last tile of a wave is peeled off, so that the
// prefetch in the loop is unconditional.
struct MixedArgs {
    const void* src[kMaxSrc];
    void* dst;
    size_t nvec;   // 16-byte vectors per source
};

template <int NSRC>
struct MixedReduceShape {
    static constexpr int kU = NSRC <= 8 ? 4 : 2;
    static constexpr size_t kTile = (size_t)kWave * kU;
};

template <int NSRC, bool NT>
__device__ __forceinline__ void mixed_reduce_load(u32x4 (&x)[MixedReduceShape<NSRC>::kU][NSRC], const MixedArgs& a,
                                                  size_t t, size_t lane)
{
    using Sh = MixedReduceShape<NSRC>;
#pragma unroll
    for (int u = 0; u < Sh::kU; ++u)
#pragma unroll
        for (int r = 0; r < NSRC; ++r)
            x[u][r] = ld<NT>(a.src[r], t * Sh::kTile + lane + (size_t)u * kWave);
}

template <int NSRC, bool NT>
__device__ __forceinline__ void mixed_reduce_store(const u32x4 (&x)[MixedReduceShape<NSRC>::kU][NSRC],
                                                   const MixedArgs& a, size_t t, size_t lane)
{
    using Sh = MixedReduceShape<NSRC>;
#pragma unroll
    for (int u = 0; u < Sh::kU; ++u) {
        u32x4 y = x[u][0];
#pragma unroll
        for (int r = 1; r < NSRC; ++r) y ^= x[u][r];
        st<NT>(a.dst, t * Sh::kTile + lane + (size_t)u * kWave, y);
    }
}

template <int NSRC, bool NT, bool PF>
__global__ __launch_bounds__(256) void k_mixed_reduce(MixedArgs a)
{
    using Sh = MixedReduceShape<NSRC>;
    constexpr int U = Sh::kU;
    const size_t waves = (size_t)gridDim.x * (blockDim.x / kWave);
    const size_t wave = (size_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const size_t lane = threadIdx.x % kWave;
    const size_t ntiles = a.nvec / Sh::kTile;
    if constexpr (PF) {
        if (wave < ntiles) {
            u32x4 xa[U][NSRC], xb[U][NSRC];
            size_t t = wave;
            size_t n = (ntiles - t + waves - 1) / waves;
            mixed_reduce_load<NSRC, NT>(xa, a, t, lane);
            for (;;) {
                if (n == 1) { mixed_reduce_store<NSRC, NT>(xa, a, t, lane); break; }
                mixed_reduce_load<NSRC, NT>(xb, a, t + waves, lane);
                mixed_reduce_store<NSRC, NT>(xa, a, t, lane);
                t += waves;
                --n;
                if (n == 1) { mixed_reduce_store<NSRC, NT>(xb, a, t, lane); break; }
                mixed_reduce_load<NSRC, NT>(xa, a, t + waves, lane);
                mixed_reduce_store<NSRC, NT>(xb, a, t, lane);
                t += waves;
                --n;
            }
        }
    } else {
        for (size_t t = wave; t < ntiles; t += waves) {
            u32x4 x[U][NSRC];
            mixed_reduce_load<NSRC, NT>(x, a, t, lane);
            mixed_reduce_store<NSRC, NT>(x, a, t, lane);
        }
    }
    if (ntiles * Sh::kTile < a.nvec && wave == ntiles % waves) {
        for (int u = 0; u < U; ++u) {
            const size_t v = ntiles * Sh::kTile + lane + (size_t)u * kWave;
            if (v >= a.nvec) break;
            u32x4 y = ld16(a.src[0], v);
            for (int r = 1; r < NSRC; ++r) y ^= ld16(a.src[r], v);
            st16(a.dst, v, y);
        }
    }
}

// narrow: K = 2 or 4; U loads per lane per tile (8 with the prefetch, as the
// quantizer's largest variant, 4 without)
template <int K, bool NT, int U>
__device__ __forceinline__ void mixed_narrow_load(u32x4 (&x)[U], const MixedArgs& a, size_t t, size_t lane)
{
#pragma unroll
    for (int u = 0; u < U; ++u)
        x[u] = ld<NT>(a.src[0], t * kWave * U + lane + (size_t)u * kWave);
}

template <int K, bool NT>
__device__ __forceinline__ void narrow_store(const MixedArgs& a, size_t v, const u32x4& x)
{
    if constexpr (K == 2) {
        u32x2 w = {x[0] ^ x[1], x[2] ^ x[3]};
        if constexpr (NT) __builtin_nontemporal_store(w, static_cast<u32x2*>(a.dst) + v);
        else static_cast<u32x2*>(a.dst)[v] = w;
    } else {
        uint32_t w = x[0] ^ x[1] ^ x[2] ^ x[3];
        if constexpr (NT) __builtin_nontemporal_store(w, static_cast<uint32_t*>(a.dst) + v);
        else static_cast<uint32_t*>(a.dst)[v] = w;
    }
}

template <int K, bool NT, int U>
__device__ __forceinline__ void mixed_narrow_store(const u32x4 (&x)[U], const MixedArgs& a, size_t t, size_t lane)
{
#pragma unroll
    for (int u = 0; u < U; ++u)
        narrow_store<K, NT>(a, t * kWave * U + lane + (size_t)u * kWave, x[u]);
}

template <int K, bool NT, bool PF>
__global__ __launch_bounds__(256) void k_mixed_narrow(MixedArgs a)
{
    constexpr int U = PF ? 8 : 4;
    constexpr size_t kTile = (size_t)kWave * U;
    const size_t waves = (size_t)gridDim.x * (blockDim.x / kWave);
    const size_t wave = (size_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const size_t lane = threadIdx.x % kWave;
    const size_t ntiles = a.nvec / kTile;
    if constexpr (PF) {
        if (wave < ntiles) {
            u32x4 xa[U], xb[U];
            size_t t = wave;
            size_t n = (ntiles - t + waves - 1) / waves;
            mixed_narrow_load<K, NT, U>(xa, a, t, lane);
            for (;;) {
                if (n == 1) { mixed_narrow_store<K, NT, U>(xa, a, t, lane); break; }
                mixed_narrow_load<K, NT, U>(xb, a, t + waves, lane);
                mixed_narrow_store<K, NT, U>(xa, a, t, lane);
                t += waves;
                --n;
                if (n == 1) { mixed_narrow_store<K, NT, U>(xb, a, t, lane); break; }
                mixed_narrow_load<K, NT, U>(xa, a, t + waves, lane);
                mixed_narrow_store<K, NT, U>(xb, a, t, lane);
                t += waves;
                --n;
            }
        }
    } else {
        for (size_t t = wave; t < ntiles; t += waves) {
            u32x4 x[U];
            mixed_narrow_load<K, NT, U>(x, a, t, lane);
            mixed_narrow_store<K, NT, U>(x, a, t, lane);
        }
    }
    if (ntiles * kTile < a.nvec && wave == ntiles % waves) {
        for (int u = 0; u < U; ++u) {
            const size_t v = ntiles * kTile + lane + (size_t)u * kWave;
            if (v >= a.nvec) break;
            narrow_store<K, false>(a, v, ld16(a.src[0], v));
        }
    }
}

// The tree step's memory pattern without its arithmetic: N streams copied,
// src[j] -> dst[j] over the same range of 16-byte vectors [v0, v1): N reads
// and N writes of the range, each stream its own allocation. LANES 1: one
// lane per vector, its N loads, then its N stores; LANES 2: two lanes per
// vector, the first half-wave copying streams 0..H-1 and the second H..N-1
// (H = ceil(N / 2)). Nontemporal loads and stores, as in the tree step.
struct StreamsArgs {
    const void* src[kMaxSrc];
    void* dst[kMaxSrc];
    size_t v0, v1;
};

template <int N, int LANES>
__global__ __launch_bounds__(256) void k_copy_streams(StreamsArgs a)
{
    const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    if constexpr (LANES == 1) {
        for (size_t v = a.v0 + gid; v < a.v1; v += stride) {
            u32x4 x[N];
#pragma unroll
            for (int r = 0; r < N; ++r) x[r] = ld16_stream(a.src[r], v);
#pragma unroll
            for (int j = 0; j < N; ++j) st16_stream(a.dst[j], v, x[j]);
        }
    } else {
        constexpr int H = (N + 1) / 2;
        const int lane = lane_id();
        const int half = lane / (kWave / 2);
        const int first = half ? H : 0;
        const int cnt = half ? N - H : H;
        const size_t vv = (gid / kWave) * (kWave / 2) + (size_t)(lane % (kWave / 2));
        for (size_t v = a.v0 + vv; v < a.v1; v += stride / 2) {
            u32x4 x[H];
#pragma unroll
            for (int r = 0; r < H; ++r)
                if (r < cnt) x[r] = ld16_stream(a.src[first + r], v);
#pragma unroll
            for (int j = 0; j < H; ++j)
                if (j < cnt) st16_stream(a.dst[first + j], v, x[j]);
        }
    }
}

using StreamsFn = void (*)(StreamsArgs);

template <int LANES, int... I>
constexpr std::array<StreamsFn, sizeof...(I)> streams_table(std::integer_sequence<int, I...>)
{
    return {{&k_copy_streams<I + 1, LANES>...}};
}

const std::array<StreamsFn, kMaxSrc> kCopyStreams[2] = {
    streams_table<1>(std::make_integer_sequence<int, kMaxSrc>{}),
    streams_table<2>(std::make_integer_sequence<int, kMaxSrc>{})};

using MixedFn = void (*)(MixedArgs);

template <bool NT, bool PF, int... I>
constexpr std::array<MixedFn, sizeof...(I)> mixed_reduce_table(std::integer_sequence<int, I...>)
{
    return {{&k_mixed_reduce<I + 1, NT, PF>...}};
}

// [prefetch][nontemporal][nsrc - 1]
const std::array<MixedFn, kMaxSrc> kMixedReduce[2][2] = {
    {mixed_reduce_table<false, false>(std::make_integer_sequence<int, kMaxSrc>{}),
     mixed_reduce_table<true, false>(std::make_integer_sequence<int, kMaxSrc>{})},
    {mixed_reduce_table<false, true>(std::make_integer_sequence<int, kMaxSrc>{}),
     mixed_reduce_table<true, true>(std::make_integer_sequence<int, kMaxSrc>{})}};
// [prefetch][K == 4][nontemporal]
const MixedFn kMixedNarrow[2][2][2] = {
    {{k_mixed_narrow<2, false, false>, k_mixed_narrow<2, true, false>},
     {k_mixed_narrow<4, false, false>, k_mixed_narrow<4, true, false>}},
    {{k_mixed_narrow<2, false, true>, k_mixed_narrow<2, true, true>},
     {k_mixed_narrow<4, false, true>, k_mixed_narrow<4, true, true>}}};

typedef void (*StreamFn)(const void*, void*, size_t, u32x4);
const StreamFn kStream[4][2] = {
    {k_stream<0, false>, k_stream<0, true>},
    {k_stream<1, false>, k_stream<1, true>},
    {k_stream<2, false>, k_stream<2, true>},
    {k_stream<3, false>, k_stream<3, false>},
};

}  // namespace
}  // namespace rx

extern "C" {

size_t rxtest_stream_sink_bytes(int wgs_per_cu)
{
    if (wgs_per_cu < 1 || wgs_per_cu > 8) return 0;
    return (size_t)rx::device_cu_count() * (size_t)wgs_per_cu * (256u / rx::kWave) * 16u;
}

rx_status_t rxtest_stream(int kind, const void* src, void* dst, size_t bytes, int wgs_per_cu,
                          int nontemporal, hipStream_t stream)
{
    if (kind < 0 || kind > 3 || wgs_per_cu < 1 || wgs_per_cu > 8) return RX_ERR_ARG;
    if (kind != 3 && (!dst || (kind != 1 && !src))) return RX_ERR_NULL;
    if (bytes % 16 || (uintptr_t)dst % 16 || (uintptr_t)src % 16) return RX_ERR_ALIGN;
    if (bytes == 0 && kind != 3) return RX_OK;
    const unsigned grid = (unsigned)(rx::device_cu_count() * wgs_per_cu);
    const rx::u32x4 pattern = {0x3F800000u, 0x40000000u, 0x40400000u, 0x40800000u};
    void* args_dst = dst;
    const void* args_src = src;
    size_t nvec = bytes / 16;
    rx::u32x4 pat = pattern;
    void* params[] = {&args_src, &args_dst, &nvec, &pat};
    const hipError_t e = hipLaunchKernel((const void*)rx::kStream[kind][nontemporal ? 1 : 0],
                                         dim3(grid), dim3(256), params, 0, stream);
    if (e != hipSuccess)
        fprintf(stderr, "librx: launch failed: %s\n", hipGetErrorName(e));
    return e == hipSuccess ? RX_OK : RX_ERR_HIP;
}

rx_status_t rxtest_stream_mixed(int kind, const void* const* srcs, int nsrc, void* dst,
                                size_t src_bytes, int wgs_per_cu, int nontemporal, int prefetch,
                                hipStream_t stream)
{
    if (kind < 0 || kind > 2 || wgs_per_cu < 1 || wgs_per_cu > 8) return RX_ERR_ARG;
    if (prefetch != 0 && prefetch != 1) return RX_ERR_ARG;
    if (nsrc < 1 || nsrc > RX_MAX_SRC || (kind != 0 && nsrc != 1)) return RX_ERR_ARG;
    if (!srcs || !dst) return RX_ERR_NULL;
    for (int j = 0; j < nsrc; ++j)
        if (!srcs[j]) return RX_ERR_NULL;
    for (int j = 0; j < nsrc; ++j)
        if ((uintptr_t)srcs[j] % 16) return RX_ERR_ALIGN;
    if (src_bytes % 16 || (uintptr_t)dst % 16) return RX_ERR_ALIGN;
    if (src_bytes == 0) return RX_OK;
    rx::MixedArgs a = {};
    for (int j = 0; j < nsrc; ++j) a.src[j] = srcs[j];
    a.dst = dst;
    a.nvec = src_bytes / 16;
    const int nt = nontemporal ? 1 : 0;
    const rx::MixedFn fn = kind == 0 ? rx::kMixedReduce[prefetch][nt][nsrc - 1]
                                     : rx::kMixedNarrow[prefetch][kind - 1][nt];
    const unsigned grid = (unsigned)(rx::device_cu_count() * wgs_per_cu);
    void* params[] = {&a};
    const hipError_t e = hipLaunchKernel((const void*)fn, dim3(grid), dim3(256), params, 0, stream);
    if (e != hipSuccess)
        fprintf(stderr, "librx: launch failed: %s\n", hipGetErrorName(e));
    return e == hipSuccess ? RX_OK : RX_ERR_HIP;
}

rx_status_t rxtest_copy_streams(const void* const* srcs, void* const* dsts, int n,
                                size_t offset_bytes, size_t bytes, int lanes, int wg,
                                hipStream_t stream)
{
    if (n < 1 || n > RX_MAX_SRC || (lanes != 1 && lanes != 2) || (wg != 64 && wg != 128 && wg != 256))
        return RX_ERR_ARG;
    if (!srcs || !dsts) return RX_ERR_NULL;
    for (int j = 0; j < n; ++j)
        if (!srcs[j] || !dsts[j]) return RX_ERR_NULL;
    for (int j = 0; j < n; ++j)
        if ((uintptr_t)srcs[j] % 16 || (uintptr_t)dsts[j] % 16) return RX_ERR_ALIGN;
    if (offset_bytes % 16 || bytes % 16) return RX_ERR_ALIGN;
    if (bytes == 0) return RX_OK;
    rx::StreamsArgs a = {};
    for (int j = 0; j < n; ++j) {
        a.src[j] = srcs[j];
        a.dst[j] = dsts[j];
    }
    a.v0 = offset_bytes / 16;
    a.v1 = a.v0 + bytes / 16;
    const size_t threads = (bytes / 16) * (size_t)lanes;
    size_t grid = (threads + (size_t)wg - 1) / (size_t)wg;
    if (grid > 65536) grid = 65536;   // grid-stride beyond
    void* params[] = {&a};
    const hipError_t e = hipLaunchKernel((const void*)rx::kCopyStreams[lanes - 1][n - 1],
                                         dim3((unsigned)grid), dim3((unsigned)wg), params, 0, stream);
    if (e != hipSuccess)
        fprintf(stderr, "librx: launch failed: %s\n", hipGetErrorName(e));
    return e == hipSuccess ? RX_OK : RX_ERR_HIP;
}

}  // extern "C"
