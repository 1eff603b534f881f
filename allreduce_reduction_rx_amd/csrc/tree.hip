// tree.hip -- DDA tree per-rank step (gfx950): reduce this rank's chunk
// across the N sources in FP32, in source order, and push it into every
// destination (RCCLX article, code-journey.com, "Core feature 1: Direct Data
// Access (DDA)", DDA Tree item; "Core feature 2", table row "Compute
// precision"). 16-byte nontemporal loads of every source, issued before the
// first add; nontemporal stores into every destination; N is a template
// parameter.
#include "reduce_common.hpp"

namespace rx {
namespace {

// Ragged end of a chunk (hi not a multiple of the vector): element-wise.
template <int DT, int N>
__device__ __forceinline__ void tree_tail(const TreeArgs& a, size_t v1, size_t gid)
{
    constexpr int VE = Elem<DT>::kVE;
    const size_t i = v1 * VE + gid;
    if (i >= a.lo && i < a.hi) {
        float z = fold_vec_tail<DT, N>(a.src, i);
#pragma unroll
        for (int j = 0; j < N; ++j)
            store_elem<DT>(a.dst[j], i, z);
    }
}

// Two lanes per 16-byte vector: the two half-waves fold the same 32 vectors
// (their loads share cache lines) and each writes half of the N
// destinations, so twice the threads share the stores. Nontemporal source
// loads and destination stores (cached ones measured 15-20% slower at
// 8 x 4 MiB). TAIL: the chunk ends in a partial vector; the instance
// without it carries no tail code (0.1 us per decode-size launch).
template <int DT, int N, bool TAIL>
__global__ __launch_bounds__(256) void k_tree(TreeArgs a)
{
    constexpr int VE = Elem<DT>::kVE;
    constexpr int H = (N + 1) / 2;        // destinations of the first half-wave
    const size_t v0 = a.lo / VE;          // lo is 16-B aligned (or == hi)
    const size_t v1 = a.hi / VE;
    const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    const int lane = lane_id();
    const int half = lane / (kWave / 2);
    const int first = half ? H : 0;
    const int cnt = half ? N - H : H;
    // wave w takes vectors 32w .. 32w + 31, both halves the same ones
    const size_t vv = (gid / kWave) * (kWave / 2) + (size_t)(lane % (kWave / 2));
    for (size_t v = v0 + vv; v < v1; v += stride / 2) {
        u32x4 y = fold_vec<DT, N, true, true>(a.src, v);
#pragma unroll
        for (int j = 0; j < H; ++j)
            if (j < cnt)
                st16_stream(a.dst[first + j], v, y);
    }
    if constexpr (TAIL)
        tree_tail<DT, N>(a, v1 > v0 ? v1 : v0, gid);
}

// Small chunks (up to one 64-thread workgroup of half-vector lanes per CU):
// each lane folds one 4-byte word (one FP32 or two BF16 elements) over all N
// sources and stores it into all N destinations; no load is issued twice.
// Four lanes per 16-byte vector spread a decode-size chunk over every CU
// (8 x 512 KiB BF16 messages, chunk 64 KiB: 2.33 -> 2.14 us against
// 8-byte lanes, which filled half the CUs; chunks of 32 and 128 KiB 7% and 3%
// faster). The grid holds a lane for every word, so there is no loop. The
// pointers' null test in the bounds test loads every source and destination
// pointer before its branch, with the range (eight in-place launches over
// 8 x 512 KiB, the one-device TREE allreduce: 19.9 -> 18.7 us). TAIL: a BF16
// chunk that ends on an odd element; its last element is folded alone.
template <int DT, int N, bool TAIL>
__global__ __launch_bounds__(256) void k_tree_word(TreeArgs a)
{
    constexpr int WE = DT == 0 ? 1 : 2;        // elements per 4-byte word
    const size_t w0 = a.lo / WE;               // lo is a vector multiple
    const size_t w1 = a.hi / WE;
    const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t w = w0 + gid;
    uint32_t m = ~0u;
#pragma unroll
    for (int r = 0; r < N; ++r) {
        const uint32_t p = ptr_nonzero(a.src[r]), q = ptr_nonzero(a.dst[r]);
        m = m < p ? m : p;
        m = m < q ? m : q;
    }
    if ((w < w1) & (m != 0)) {
        uint32_t x[N];
#pragma unroll
        for (int r = 0; r < N; ++r)
            x[r] = __builtin_nontemporal_load(static_cast<const uint32_t*>(a.src[r]) + w);
        uint32_t y;
        if constexpr (DT == 0) {
            float acc = bits_f32(x[0]);
#pragma unroll
            for (int r = 1; r < N; ++r)
                acc = acc + bits_f32(x[r]);
            y = __builtin_bit_cast(uint32_t, acc);
        } else {
            float lo = bf16_lo(x[0]);
            float hi = bf16_hi(x[0]);
#pragma unroll
            for (int r = 1; r < N; ++r) {
                lo = lo + bf16_lo(x[r]);
                hi = hi + bf16_hi(x[r]);
            }
            y = pack_bf16(lo, hi);
        }
#pragma unroll
        for (int j = 0; j < N; ++j)
            __builtin_nontemporal_store(y, static_cast<uint32_t*>(a.dst[j]) + w);
    }
    if constexpr (TAIL) {
        const size_t i = (w1 > w0 ? w1 : w0) * WE + gid;
        if (i >= a.lo && i < a.hi) {
            const float z = fold_vec_tail<DT, N>(a.src, i);
#pragma unroll
            for (int j = 0; j < N; ++j)
                store_elem<DT>(a.dst[j], i, z);
        }
    }
}

// Large BF16 chunks, large FP32 chunks from 64 tiles per CU, and chunks of
// either type of 6 to 8 tiles per CU (a wave per tile; see launch_tree):
// whole tiles of 64 vectors (one per lane) from lo; the N loads of a lane
// first, then the fold, then its N stores; no bounds check in the loop (the
// rest of the chunk goes to k_tree). Large chunks launch four 64-thread
// workgroups per CU: 8 x 16M BF16 in place (the one-device FLAT allreduce)
// 97.7 -> 89.6 us, 8 x 256M 1579 -> 1524 us, against 2-vector tiles with
// bounds checks in one 256-thread workgroup per CU.
template <int DT, int N>
__global__ __launch_bounds__(256) void k_tree_whole(TreeArgs a)
{
    constexpr int VE = Elem<DT>::kVE;
    const int lane = lane_id();
    const uint32_t wave_in_wg = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const size_t wave = (size_t)blockIdx.x * (blockDim.x / kWave) + wave_in_wg;
    const size_t nwaves = (size_t)gridDim.x * (blockDim.x / kWave);
    const size_t v0 = a.lo / VE;
    const size_t ntiles = (a.hi - a.lo) / VE / kWave;
    for (size_t t = wave; t < ntiles; t += nwaves) {
        const size_t v = v0 + t * kWave + lane;
        u32x4 x[N];
#pragma unroll
        for (int r = 0; r < N; ++r)
            x[r] = ld16_stream(a.src[r], v);
        const u32x4 y = fold_regs<DT, N>(x);
#pragma unroll
        for (int j = 0; j < N; ++j)
            st16_stream(a.dst[j], v, y);
    }
}

using TreeFn = void (*)(TreeArgs);

template <int DT, bool TAIL, int... I>
constexpr std::array<TreeFn, sizeof...(I)> tree_table(std::integer_sequence<int, I...>)
{
    return {{&k_tree<DT, I + 1, TAIL>...}};
}
template <int DT, bool TAIL, int... I>
constexpr std::array<TreeFn, sizeof...(I)> tree_word_table(std::integer_sequence<int, I...>)
{
    return {{&k_tree_word<DT, I + 1, TAIL>...}};
}
template <int DT, int... I>
constexpr std::array<TreeFn, sizeof...(I)> tree_whole_table(std::integer_sequence<int, I...>)
{
    return {{&k_tree_whole<DT, I + 1>...}};
}


// [dtype][tail][nsrc - 1]
const std::array<TreeFn, kMaxSrc> kTree[2][2] = {
    {tree_table<0, false>(std::make_integer_sequence<int, kMaxSrc>{}),
     tree_table<0, true>(std::make_integer_sequence<int, kMaxSrc>{})},
    {tree_table<1, false>(std::make_integer_sequence<int, kMaxSrc>{}),
     tree_table<1, true>(std::make_integer_sequence<int, kMaxSrc>{})}};
// [dtype][tail][nsrc - 1]; tail: a BF16 chunk ending on an odd element
const std::array<TreeFn, kMaxSrc> kTreeWord[2][2] = {
    {tree_word_table<0, false>(std::make_integer_sequence<int, kMaxSrc>{}),
     tree_word_table<0, true>(std::make_integer_sequence<int, kMaxSrc>{})},
    {tree_word_table<1, false>(std::make_integer_sequence<int, kMaxSrc>{}),
     tree_word_table<1, true>(std::make_integer_sequence<int, kMaxSrc>{})}};
// [dtype][nsrc - 1]: medium chunks of either type, large BF16 chunks, large
// FP32 chunks from 64 tiles per CU
const std::array<TreeFn, kMaxSrc> kTreeWhole[2] = {tree_whole_table<0>(std::make_integer_sequence<int, kMaxSrc>{}),
                                                   tree_whole_table<1>(std::make_integer_sequence<int, kMaxSrc>{})};

// Decode-size chunks run 64-thread workgroups (at 8 x 4 MiB, 2.98 us
// against 3.06 us with 128 threads).
LaunchPolicy policy_tree() { return {64u, 256u, 1u}; }
LaunchPolicy policy_tree_whole() { return {64u, 64u, 4u}; }

}  // namespace

hipError_t launch_tree(const TreeArgs& a, int nsrc, int dtype, hipStream_t s)
{
    const int ve = dtype == 0 ? 4 : 8;
    const size_t nvec = (a.hi - a.lo) / ve;
    const bool small = small_job(nvec);
    const size_t cus = (size_t)device_cu_count();
    const size_t tiles = nvec / kWave;
    // Chunks of 6 to 8 whole 64-vector tiles per CU (around the decode-size
    // threshold): k_tree_whole with a wave for every tile, 64-thread
    // workgroups, 256-thread ones from 8 tiles per CU. Against the
    // two-lanes-per-vector kernel below 8 and the grid-stride launch at 8,
    // for 2, 4 and 8 sources of either type: 2-27% faster (8 sources, 8
    // tiles per CU: BF16 8.28 -> 6.68 us, FP32 8.62 -> 6.96); at 4-5 tiles
    // per CU and at 10 and more it was not faster.
    const bool medium = tiles >= 6 * cus && tiles <= 8 * cus;
    // Large FP32 chunks from 64 tiles per CU also take k_tree_whole (8 x 32M
    // FP32 46.5 -> 45.4 us, 8 x 64M 93.5 -> 90.4; at 48 tiles per CU and
    // below k_tree was as fast or up to 2% faster)
    const bool whole = medium || (!small && (dtype != 0 || tiles >= 64 * cus));
    dim3 grid, block;
    if (whole) {
        // medium chunks, large BF16 chunks, large FP32 chunks from 64 tiles
        // per CU: whole tiles of 64 vectors, then the rest of the chunk
        // (fewer than 64 vectors and the element tail) in k_tree
        if (medium) {
            const unsigned wg = tiles >= 8 * cus ? 256u : 64u;
            grid = dim3((unsigned)((tiles * kWave + wg - 1) / wg));
            block = dim3(wg);
        } else {
            launch_geometry(tiles * kWave, false, policy_tree_whole(), grid, block);
        }
        TreeArgs arg = a;
        arg.hi = a.lo + tiles * kWave * ve;
        void* params[] = {&arg};
        const hipError_t e = launch_logged(medium ? "k_tree_whole (medium)" : "k_tree_whole",
                                           (const void*)kTreeWhole[dtype][nsrc - 1], grid, block, params, s);
        if (e != hipSuccess || arg.hi == a.hi)
            return e;
        TreeArgs rest = a;
        rest.lo = arg.hi;                                  // a vector multiple
        const int tail = rest.hi % (size_t)ve != 0 ? 1 : 0;
        launch_geometry((rest.hi - rest.lo + ve - 1) / ve, true, policy_tree(), grid, block);
        void* rparams[] = {&rest};
        return launch_logged("k_tree (rest)", (const void*)kTree[dtype][tail][nsrc - 1], grid, block, rparams, s);
    }
    TreeArgs arg = a;
    void* params[] = {&arg};
    // small chunks: 4-byte-word lanes while the words fit six waves per CU
    // (8 x 1M BF16, chunk 128K elements: 2.65 -> 2.41 us, chunk 192K 2.78 ->
    // 2.63; at eight waves per CU, 8 x 2M BF16, two lanes per vector were
    // faster, 2.97 against 3.16 us), two lanes per vector above that; a
    // small launch's grid is not capped, so k_tree_word gets a lane for
    // every word
    if (small && 4 * nvec <= (size_t)6 * kWave * cus) {
        const size_t we = dtype == 0 ? 1 : 2;            // elements per word
        const size_t words = a.hi / we - a.lo / we;      // lo is a vector multiple
        const int wtail = a.hi % we != 0 ? 1 : 0;
        launch_geometry(words, true, policy_tree(), grid, block);
        if ((size_t)grid.x * block.x < words)
            return hipErrorInvalidConfiguration;
        return launch_logged("k_tree_word", (const void*)kTreeWord[dtype][wtail][nsrc - 1], grid, block, params, s);
    }
    const int tail = a.hi % (size_t)ve != 0 ? 1 : 0;   // lo is a vector multiple
    launch_geometry(small ? 2 * nvec : nvec, small, policy_tree(), grid, block);
    return launch_logged("k_tree", (const void*)kTree[dtype][tail][nsrc - 1], grid, block, params, s);
}

}  // namespace rx
