// reduce.hip -- DDA flat local reduce (gfx950).
//
// DDA flat: each rank reads all peers' buffers directly and reduces locally
// (RCCLX article, code-journey.com, "Core feature 1: Direct Data Access
// (DDA)", DDA Flat item). Sums are FP32 ("Core feature 2", table row
// "Compute precision"), folded in source order 0..N-1.
//
// An HBM-bound stream: 16-byte nontemporal loads of every source (all N
// issued before the first add), FP32 adds, 16-byte stores. N is a template
// parameter, so the source loop unrolls and the pointer table is read with
// scalar loads from the kernarg segment.
#include "reduce_common.hpp"

namespace rx {
namespace {

// Decode-size messages: one 16-byte output vector per thread.
template <int DT, int N>
__global__ __launch_bounds__(256) void k_reduce_flat(FlatArgs a)
{
    constexpr int VE = Elem<DT>::kVE;
    const size_t nvec = a.count / VE;
    const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t v = gid; v < nvec; v += stride)
        st16(a.dst, v, fold_vec<DT, N, true>(a.src, v));
    const size_t i = nvec * VE + gid;
    if (i < a.count)
        store_elem<DT>(a.dst, i, fold_vec_tail<DT, N>(a.src, i));
}

// Large messages: each wave takes tiles of U x 64 vectors (vector u * 64 +
// lane of the tile), loads all sources of all U vectors, then issues its U
// nontemporal stores back to back. Batching the writes of a wave measured
// ~5% faster on MI355X than one store after every fold.
template <int DT, int N>
__global__ __launch_bounds__(256) void k_reduce_flat_tiles(FlatArgs a)
{
    constexpr int VE = Elem<DT>::kVE;
    constexpr int U = N <= 8 ? 4 : 2;
    const int lane = lane_id();
    const uint32_t wave_in_wg = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const size_t wave = (size_t)blockIdx.x * (blockDim.x / kWave) + wave_in_wg;
    const size_t nwaves = (size_t)gridDim.x * (blockDim.x / kWave);
    const size_t nvec = a.count / VE;
    const size_t ntiles = (nvec + (size_t)U * kWave - 1) / ((size_t)U * kWave);
    for (size_t t = wave; t < ntiles; t += nwaves) {
        const size_t base = t * U * kWave + lane;
        u32x4 y[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (base + u * kWave < nvec)
                y[u] = fold_vec<DT, N, true>(a.src, base + u * kWave);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (base + u * kWave < nvec)
                st16_stream(a.dst, base + u * kWave, y[u]);
    }
    const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t i = nvec * VE + gid;
    if (i < a.count)
        store_elem<DT>(a.dst, i, fold_vec_tail<DT, N>(a.src, i));
}

// Large messages, whole tiles of 4 x 64 vectors only (count a multiple of the
// tile; the rest of the message goes to k_reduce_flat): the loads of all N
// sources of the 4 vectors are issued first, then the folds, then the 4
// stores. The bounds checks inside k_reduce_flat_tiles' tile loop make each
// vector's loads a round trip of their own, which costs most where a tile
// holds few loads: 2 x 16M FP32 46.7 -> 32.2 us, 2 x 64M BF16 95.6 -> 62.7,
// 4 x 64M BF16 115.8 -> 109.4, 8 x 4M FP32 27.5 -> 24.6, 8 x 16M FP32
// 99.7 -> 98.4. With more sources in BF16 the checked kernel measured the
// same or faster (8 x 64M BF16 197.7 against 201.3 us) and stays.
template <int DT, int N>
__global__ __launch_bounds__(256) void k_reduce_flat_whole(FlatArgs a)
{
    constexpr int VE = Elem<DT>::kVE;
    constexpr int U = 4;
    const int lane = lane_id();
    const uint32_t wave_in_wg = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const size_t wave = (size_t)blockIdx.x * (blockDim.x / kWave) + wave_in_wg;
    const size_t nwaves = (size_t)gridDim.x * (blockDim.x / kWave);
    const size_t ntiles = a.count / VE / ((size_t)U * kWave);
    for (size_t t = wave; t < ntiles; t += nwaves) {
        const size_t base = t * U * kWave + lane;
        u32x4 x[U][N];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < N; ++r)
                x[u][r] = ld16_stream(a.src[r], base + u * kWave);
        u32x4 y[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            y[u] = fold_regs<DT, N>(x[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
            st16_stream(a.dst, base + u * kWave, y[u]);
    }
}

using FlatFn = void (*)(FlatArgs);

template <int DT, int... I>
constexpr std::array<FlatFn, sizeof...(I)> flat_table(std::integer_sequence<int, I...>)
{
    return {{&k_reduce_flat<DT, I + 1>...}};
}
template <int DT, int... I>
constexpr std::array<FlatFn, sizeof...(I)> flat_tiles_table(std::integer_sequence<int, I...>)
{
    return {{&k_reduce_flat_tiles<DT, I + 1>...}};
}
template <int DT, int... I>
constexpr std::array<FlatFn, sizeof...(I)> flat_whole_table(std::integer_sequence<int, I...>)
{
    return {{&k_reduce_flat_whole<DT, I + 1>...}};
}
const std::array<FlatFn, kMaxSrc> kFlat[2] = {
    flat_table<0>(std::make_integer_sequence<int, kMaxSrc>{}),
    flat_table<1>(std::make_integer_sequence<int, kMaxSrc>{})};
const std::array<FlatFn, kMaxSrc> kFlatTiles[2] = {
    flat_tiles_table<0>(std::make_integer_sequence<int, kMaxSrc>{}),
    flat_tiles_table<1>(std::make_integer_sequence<int, kMaxSrc>{})};
// whole-tile kernel: N <= 8 (FP32) and N <= 4 (BF16) are launched for large
// messages, N <= 8 of either type for medium ones
constexpr int kFlatWholeMax = 8;
const std::array<FlatFn, kFlatWholeMax> kFlatWhole[2] = {
    flat_whole_table<0>(std::make_integer_sequence<int, kFlatWholeMax>{}),
    flat_whole_table<1>(std::make_integer_sequence<int, kFlatWholeMax>{})};
// One thread per 16-byte output vector. Large messages run one 256-thread
// workgroup per CU with a grid-stride
// loop: on MI355X a narrow window of in-flight addresses measured up to 20%
// faster than filling every CU with 8 workgroups.
LaunchPolicy policy_flat() { return {128u, 256u, 1u}; }
}  // namespace

hipError_t launch_reduce_flat(const FlatArgs& a, int nsrc, int dtype, hipStream_t s)
{
    const int ve = dtype == 0 ? 4 : 8;
    const size_t nvec = a.count / ve;
    const bool small = small_job(nvec);
    const size_t cus = (size_t)device_cu_count();
    dim3 grid, block;
    // Medium messages (up to 16 whole tiles per CU): the whole-tile kernel
    // with a wave for every tile, in workgroups small enough that every CU
    // gets one (8 sources: 8 x 1M BF16 6.18 -> 4.83 us, 8 x 4M BF16 14.99 ->
    // 14.01, 8 x 2M FP32 13.04 -> 12.80; 2 and 4 sources 0-14% faster; against
    // one workgroup per CU striding over the tiles). From 32 tiles per CU the
    // large policy below is as fast or faster (8 x 16M BF16 49.2 us against
    // 50.3 with a wave per tile).
    const size_t whole_tiles = nvec / (4 * kWave);
    const bool medium = !small && nsrc <= kFlatWholeMax && whole_tiles <= 16 * cus;
    const bool whole = medium || (!small && (nsrc <= 4 || (dtype == 0 && nsrc <= kFlatWholeMax)));
    if (whole) {
        // whole tiles of 4 x 64 vectors, then the rest of the message (less
        // than one tile) in the decode-size kernel over offset pointers
        const size_t tile_elems = (size_t)4 * kWave * ve;
        const size_t tiles = a.count / tile_elems;
        if (medium) {
            const unsigned wg = tiles >= 4 * cus ? 256u : tiles >= 2 * cus ? 128u : 64u;
            grid = dim3((unsigned)((tiles * kWave + wg - 1) / wg));
            block = dim3(wg);
        } else {
            launch_geometry(tiles * kWave, false, policy_flat(), grid, block);   // a wave per tile
        }
        FlatArgs arg = a;
        arg.count = tiles * tile_elems;
        void* params[] = {&arg};
        const hipError_t e = launch_logged("k_reduce_flat_whole", (const void*)kFlatWhole[dtype][nsrc - 1], grid,
                                           block, params, s);
        if (e != hipSuccess || a.count == arg.count)
            return e;
        const size_t done = arg.count * (dtype == 0 ? 4 : 2);   // bytes
        FlatArgs rest = a;
        for (int j = 0; j < nsrc; ++j)
            rest.src[j] = static_cast<const uint8_t*>(a.src[j]) + done;
        rest.dst = static_cast<uint8_t*>(a.dst) + done;
        rest.count = a.count - arg.count;
        launch_geometry((rest.count + ve - 1) / ve, true, policy_flat(), grid, block);
        void* rparams[] = {&rest};
        return launch_logged("k_reduce_flat (rest)", (const void*)kFlat[dtype][nsrc - 1], grid, block, rparams,
                             s);
    }
    launch_geometry(nvec, small, policy_flat(), grid, block);
    FlatArgs arg = a;
    void* params[] = {&arg};
    const FlatFn fn = small ? kFlat[dtype][nsrc - 1] : kFlatTiles[dtype][nsrc - 1];
    return launch_logged(small ? "k_reduce_flat" : "k_reduce_flat_tiles", (const void*)fn, grid,
                         block, params, s);
}

}  // namespace rx
