// rx_internal.hpp -- host-side declarations shared by the entry points
// (api.hip) and the kernel translation units. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rx {

constexpr int kMaxSrc = 16;

// Kernel arguments are passed by value, so the pointer tables travel in the
// kernarg segment and the caller's host arrays can be freed on return.
struct FlatArgs {
    const void* src[kMaxSrc];
    void* dst;
    size_t count;     // elements
};

struct TreeArgs {
    const void* src[kMaxSrc];
    void* dst[kMaxSrc];
    size_t lo, hi;    // element range of this rank's chunk
};

struct QuantArgs {
    const void* src[kMaxSrc];
    void* codes[kMaxSrc];
    float* scales[kMaxSrc];
    size_t count;     // elements per source
    int nsrc;
};

struct DrrArgs {
    const void* codes[kMaxSrc];
    const float* scales[kMaxSrc];
    void* out_codes[kMaxSrc];    // REQUANT: nout code buffers (message-indexed)
    float* out_scales[kMaxSrc];  // REQUANT: nout scale buffers (block-indexed)
    void* out_hp;                // SUM: required; REQUANT: optional
    void* out_hps[kMaxSrc];      // REQUANT to every rank's buffer: N outputs
    size_t lo, hi;               // element range processed; lo is a block multiple
    int nout;                    // REQUANT: destinations that receive the result
    int block;                   // elements per scale block
    int hp_bf16;                 // out_hp element type: 1 = BF16, 0 = FP32
    int xcd_ranges;              // 0: plain order; 1: each XCD takes a contiguous
                                 // range of workgroups; R > 1: one tile per 64-thread
                                 // workgroup, XCD x takes tiles [x R, x R + R)
};

struct AllreduceLpArgs {
    void* buf[kMaxSrc];          // the ranks' buffers, read and overwritten
    size_t count;                // elements per buffer
    int xcd_ranges;              // 1: each XCD takes a contiguous range of tiles
};

// Launch geometry helper: number of compute units of the current device
// (cached per device on first use).
int device_cu_count();

// How a kernel spreads `threads` work items (one per 16-byte vector, or 64
// per wave tile) over the GPU. Decode-size jobs (`small`) get one work item
// per thread in `wg_small`-thread workgroups, so that even a 512 KiB message
// reaches every CU; large jobs use `wg_large` threads and at most
// `max_wgs_per_cu` workgroups per CU with a grid-stride loop (fewer waves in
// flight keep the HBM access window narrow).
struct LaunchPolicy {
    unsigned wg_small;
    unsigned wg_large;
    unsigned max_wgs_per_cu;
};

// Jobs below this many threads per CU count as decode-size.
constexpr size_t kSmallThreadsPerCu = 512;

// Quantizer and dequant-reduce-requant: below this many large-variant wave
// tiles per CU a message counts as decode-size and takes the narrow variant.
constexpr size_t kSmallTilesPerCu = 8;

void launch_geometry(size_t threads, bool small, const LaunchPolicy& p, dim3& grid, dim3& block);

// RX_DEBUG=1 in the environment (read once): every launch prints its
// kernel, grid and workgroup size to stderr before it is launched.
bool debug_enabled();
hipError_t launch_logged(const char* what, const void* fn, dim3 grid, dim3 block, void** params,
                         hipStream_t s);

// Launchers (return the hipError_t of the launch). dtype: 0 FP32, 1 BF16.
// fmt: 0 E4M3, 1 E5M2.
hipError_t launch_reduce_flat(const FlatArgs& a, int nsrc, int dtype, hipStream_t s);
hipError_t launch_tree(const TreeArgs& a, int nsrc, int dtype, hipStream_t s);
hipError_t launch_quant(const QuantArgs& a, int src_dtype, int fmt, int block, hipStream_t s);
hipError_t launch_drr(const DrrArgs& a, int nsrc, int fmt, bool requant, hipStream_t s);
// One-pass low-precision allreduce of the ranks' buffers (block <= 64
// 16-byte vectors: allreduce_lp_fits), block 32..512.
bool allreduce_lp_fits(int dtype, int block);
hipError_t launch_allreduce_lp(const AllreduceLpArgs& a, int nsrc, int dtype, int fmt, int block,
                               hipStream_t s);

}  // namespace rx
