// api.hip -- the C ABI of librx: argument validation, kernel-argument
// packing and launch. Every check runs before the first HIP call, so an
// invalid call enqueues nothing. The operations are documented in rx.h.
#include <atomic>
#include <mutex>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "rx.h"
#include "rx_internal.hpp"

namespace rx {

int device_cu_count()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        dev = 0;
    if (dev < 64) {
        int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0)
            return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (dev < 64)
        cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

void launch_geometry(size_t threads, bool small, const LaunchPolicy& p, dim3& grid, dim3& block)
{
    const size_t cus = (size_t)device_cu_count();
    if (threads == 0)
        threads = 1;
    const unsigned wg = small ? p.wg_small : p.wg_large;
    size_t blocks = (threads + wg - 1) / wg;
    if (!small && blocks > cus * p.max_wgs_per_cu)
        blocks = cus * p.max_wgs_per_cu;
    grid = dim3((unsigned)blocks);
    block = dim3(wg);
}

bool debug_enabled()
{
    static const bool debug = [] {
        const char* d = getenv("RX_DEBUG");
        return d && d[0] == '1';
    }();
    return debug;
}

hipError_t launch_logged(const char* what, const void* fn, dim3 grid, dim3 block, void** params,
                         hipStream_t s)
{
    if (debug_enabled())
        fprintf(stderr, "librx: %s grid %u x %u threads, stream %p\n", what, grid.x, block.x,
                (void*)s);
    return hipLaunchKernel(fn, grid, block, params, 0, s);
}

}  // namespace rx

// Scratch of rx_allreduce_local_noalloc: the low-precision algorithm's codes
// and scales live here instead of in a caller's workspace. One copy per
// device (the code object's data is instantiated on every device the library
// runs on), held until the process ends. Host code never passes `scratch`
// itself to a kernel or a copy (on the host the name stands for a host-side
// stand-in, not a device address): it uses the address hipGetSymbolAddress
// returns for the current device, looked up once per device (scratch_ptr).
static __device__ __align__(256) uint8_t scratch[RX_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kMaxCount = (size_t)1 << 38;  // elements per buffer

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
bool hp_type(rx_dtype_t t) { return t == RX_FP32 || t == RX_BF16; }
bool fp8_type(rx_dtype_t t) { return t == RX_FP8_E4M3 || t == RX_FP8_E5M2; }
bool valid_block(int b) { return b >= 32 && b <= 1024 && (b & (b - 1)) == 0; }

// A failed launch is always reported on stderr with the HIP error's name.
rx_status_t launched(hipError_t e)
{
    if (e == hipSuccess)
        return RX_OK;
    fprintf(stderr, "librx: launch failed: %s (%s)\n", hipGetErrorName(e), hipGetErrorString(e));
    return RX_ERR_HIP;
}

// Shared checks of a source-pointer array: NULL array / entries, alignment.
rx_status_t check_ptrs(const void* const* p, int n, bool align16)
{
    if (!p)
        return RX_ERR_NULL;
    for (int j = 0; j < n; ++j)
        if (!p[j])
            return RX_ERR_NULL;
    for (int j = 0; j < n; ++j)
        if (align16 ? !aligned16(p[j]) : !aligned4(p[j]))
            return RX_ERR_ALIGN;
    return RX_OK;
}

size_t round256(size_t n) { return (n + 255u) / 256u * 256u; }

size_t lp_chunk_len(size_t count, int nsrc, int block)
{
    size_t c = (count + (size_t)nsrc - 1) / (size_t)nsrc;
    return (c + (size_t)block - 1) / (size_t)block * (size_t)block;
}

size_t tree_chunk_len(size_t count, int nsrc, rx_dtype_t dtype)
{
    const size_t ve = dtype == RX_BF16 ? 8 : 4;
    size_t c = (count + (size_t)nsrc - 1) / (size_t)nsrc;
    return (c + ve - 1) / ve * ve;
}

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];  // per device, set once
std::mutex g_scratch_mutex;

// This device's scratch address, or nullptr when the device cannot be
// queried or the lookup fails (reported as RX_ERR_HIP).
void* scratch_ptr()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p)
        return p;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p)
        return p;
    void* q = nullptr;
    const hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !q) {
        fprintf(stderr, "librx: scratch lookup on device %d failed: %s\n", dev, hipGetErrorName(e));
        return nullptr;
    }
    g_scratch_ptr[dev].store(q, std::memory_order_release);
    return q;
}

rx_status_t scratch_too_small(size_t need)
{
    if (rx::debug_enabled())
        fprintf(stderr, "librx: the call needs %zu bytes of scratch, the library holds %zu\n",
                need, (size_t)RX_NOALLOC_SCRATCH_BYTES);
    return RX_ERR_SCRATCH;
}

// rx_allreduce_local and rx_allreduce_local_noalloc. With use_scratch the
// low-precision algorithm's codes and scales go to this device's scratch
// array (looked up after validation, before the first launch) instead of the
// caller's workspace; nothing else differs.
rx_status_t allreduce_local_impl(void* const* bufs, int nsrc, size_t count, rx_dtype_t dtype,
                                 rx_algo_t algo, rx_dtype_t fp8_dtype, int block,
                                 void* workspace, size_t workspace_bytes, bool use_scratch,
                                 hipStream_t stream)
{
    if (!bufs)
        return RX_ERR_NULL;
    if (nsrc < 1 || nsrc > RX_MAX_SRC || count > kMaxCount || algo < RX_ALGO_AUTO ||
        algo > RX_ALGO_LOWPREC)
        return RX_ERR_ARG;
    if (!hp_type(dtype))
        return RX_ERR_DTYPE;
    rx_status_t st = check_ptrs(reinterpret_cast<const void* const*>(bufs), nsrc, true);
    if (st != RX_OK)
        return st;
    const size_t esz = dtype == RX_BF16 ? 2 : 4;
    if (algo == RX_ALGO_AUTO) {
        const char* en = getenv("RX_LOW_PRECISION_ENABLE");
        const bool lp = en && en[0] == '1' && en[1] == '\0' && count * esz >= ((size_t)16 << 20);
        algo = lp ? RX_ALGO_LOWPREC : RX_ALGO_FLAT;
    }
    size_t need = 0;
    if (algo == RX_ALGO_LOWPREC) {
        if (!valid_block(block))
            return RX_ERR_ARG;
        if ((count / 256 + 1) * (size_t)nsrc >= ((size_t)1 << 32))   // the quantizer's limit
            return RX_ERR_ARG;
        if (!fp8_type(fp8_dtype))
            return RX_ERR_DTYPE;
        need = rx_allreduce_local_workspace(nsrc, count, block);
        if (use_scratch) {
            // only the two-pass form (blocks beyond the one-pass limit)
            // keeps codes and scales in the scratch
            if (!rx::allreduce_lp_fits(dtype == RX_BF16 ? 1 : 0, block) && need > workspace_bytes)
                return scratch_too_small(need);
        } else {
            if (!workspace)
                return RX_ERR_NULL;
            if (((uintptr_t)workspace & 255u) != 0)
                return RX_ERR_ALIGN;
            if (workspace_bytes < need)
                return RX_ERR_ARG;
        }
    }
    if (use_scratch) {
        // the set-up runs on every call (also count == 0 and the algorithms
        // that need no scratch), so a caller can make it happen outside a
        // stream capture; after the first call on a device it is a lookup
        workspace = scratch_ptr();
        if (!workspace)
            return RX_ERR_HIP;
    }
    if (count == 0)
        return RX_OK;
    const int dt = dtype == RX_BF16 ? 1 : 0;

    if (algo == RX_ALGO_FLAT || algo == RX_ALGO_TREE) {
        rx::TreeArgs a = {};
        for (int j = 0; j < nsrc; ++j) {
            a.src[j] = bufs[j];
            a.dst[j] = bufs[j];
        }
        if (algo == RX_ALGO_FLAT) {
            a.lo = 0;
            a.hi = count;
            return launched(rx::launch_tree(a, nsrc, dt, stream));
        }
        for (int k = 0; k < nsrc; ++k) {
            rx_tree_chunk(count, nsrc, dtype, k, &a.lo, &a.hi);
            if (a.lo >= a.hi)
                continue;
            rx_status_t r = launched(rx::launch_tree(a, nsrc, dt, stream));
            if (r != RX_OK)
                return r;
        }
        return RX_OK;
    }

    const int fmt = fp8_dtype == RX_FP8_E5M2 ? 1 : 0;
    if (rx::allreduce_lp_fits(dt, block)) {
        // a block lies in one wave's lanes: every rank's quantization, the
        // reduction, the requantization and every rank's dequantization in
        // one pass, the codes kept in registers (the workspace is not used)
        rx::AllreduceLpArgs l = {};
        for (int j = 0; j < nsrc; ++j)
            l.buf[j] = bufs[j];
        l.count = count;
        return launched(rx::launch_allreduce_lp(l, nsrc, dt, fmt, block, stream));
    }

    // larger blocks: codes and scales of every rank in the workspace
    const size_t nb = (count + (size_t)block - 1) / (size_t)block;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    void* codes[RX_MAX_SRC];
    float* scales[RX_MAX_SRC];
    for (int j = 0; j < nsrc; ++j) {
        codes[j] = ws + (size_t)j * round256(count);
        scales[j] = reinterpret_cast<float*>(ws + (size_t)nsrc * round256(count) +
                                             (size_t)j * round256(nb * sizeof(float)));
    }
    rx::QuantArgs q = {};
    for (int j = 0; j < nsrc; ++j) {
        q.src[j] = bufs[j];
        q.codes[j] = codes[j];
        q.scales[j] = scales[j];
    }
    q.count = count;
    q.nsrc = nsrc;
    rx_status_t r = launched(rx::launch_quant(q, dt, fmt, block, stream));
    if (r != RX_OK)
        return r;
    // On one device the nsrc ranks' low-precision tree steps (each reducing
    // and requantizing its chunk) and their dequantizations of the gathered
    // FP8 message collapse into one pass: reduce, requantize, dequantize, and
    // write the result into every rank's buffer.
    rx::DrrArgs d = {};
    for (int j = 0; j < nsrc; ++j) {
        d.codes[j] = codes[j];
        d.scales[j] = scales[j];
        d.out_hps[j] = bufs[j];
    }
    d.lo = 0;
    d.hi = count;
    d.block = block;
    d.hp_bf16 = dt;
    r = launched(rx::launch_drr(d, nsrc, fmt, true, stream));
    if (r != RX_OK)
        return r;
    return RX_OK;
}

}  // namespace

extern "C" {

const char* rx_status_string(rx_status_t s)
{
    switch (s) {
    case RX_OK: return "RX_OK";
    case RX_ERR_NULL: return "RX_ERR_NULL: a required pointer is NULL";
    case RX_ERR_ARG: return "RX_ERR_ARG: invalid nsrc, rank, block, mode or count";
    case RX_ERR_DTYPE: return "RX_ERR_DTYPE: dtype not supported by this operation";
    case RX_ERR_ALIGN: return "RX_ERR_ALIGN: buffer misaligned (16 B data, 4 B scales)";
    case RX_ERR_HIP: return "RX_ERR_HIP: the HIP runtime rejected the launch";
    case RX_ERR_SCRATCH: return "RX_ERR_SCRATCH: the call needs more than the library's scratch";
    }
    return "unknown rx_status_t";
}

rx_status_t rx_reduce_flat(const void* const* srcs, int nsrc, size_t count,
                           rx_dtype_t dtype, void* dst, hipStream_t stream)
{
    if (!srcs || !dst)
        return RX_ERR_NULL;
    if (nsrc < 1 || nsrc > RX_MAX_SRC || count > kMaxCount)
        return RX_ERR_ARG;
    if (!hp_type(dtype))
        return RX_ERR_DTYPE;
    rx_status_t st = check_ptrs(srcs, nsrc, true);
    if (st != RX_OK)
        return st;
    if (!aligned16(dst))
        return RX_ERR_ALIGN;
    if (count == 0)
        return RX_OK;
    rx::FlatArgs a = {};
    for (int j = 0; j < nsrc; ++j)
        a.src[j] = srcs[j];
    a.dst = dst;
    a.count = count;
    return launched(rx::launch_reduce_flat(a, nsrc, dtype == RX_BF16 ? 1 : 0, stream));
}

rx_status_t rx_tree_chunk(size_t count, int nsrc, rx_dtype_t dtype, int rank,
                          size_t* lo, size_t* hi)
{
    if (!lo || !hi)
        return RX_ERR_NULL;
    if (nsrc < 1 || nsrc > RX_MAX_SRC || rank < 0 || rank >= nsrc || count > kMaxCount)
        return RX_ERR_ARG;
    if (!hp_type(dtype))
        return RX_ERR_DTYPE;
    const size_t c = tree_chunk_len(count, nsrc, dtype);
    size_t a = (size_t)rank * c;
    if (a > count) a = count;
    size_t b = a + c;
    if (b > count) b = count;
    *lo = a;
    *hi = b;
    return RX_OK;
}

rx_status_t rx_reduce_scatter_chunk_bcast(const void* const* srcs, int nsrc,
                                          size_t count, rx_dtype_t dtype,
                                          int rank, void* const* dsts,
                                          hipStream_t stream)
{
    if (!srcs || !dsts)
        return RX_ERR_NULL;
    if (nsrc < 1 || nsrc > RX_MAX_SRC || rank < 0 || rank >= nsrc || count > kMaxCount)
        return RX_ERR_ARG;
    if (!hp_type(dtype))
        return RX_ERR_DTYPE;
    rx_status_t st = check_ptrs(srcs, nsrc, true);
    if (st != RX_OK)
        return st;
    st = check_ptrs(reinterpret_cast<const void* const*>(dsts), nsrc, true);
    if (st != RX_OK)
        return st;
    size_t lo = 0, hi = 0;
    rx_tree_chunk(count, nsrc, dtype, rank, &lo, &hi);
    if (lo >= hi)
        return RX_OK;
    rx::TreeArgs a = {};
    for (int j = 0; j < nsrc; ++j) {
        a.src[j] = srcs[j];
        a.dst[j] = dsts[j];
    }
    a.lo = lo;
    a.hi = hi;
    return launched(rx::launch_tree(a, nsrc, dtype == RX_BF16 ? 1 : 0, stream));
}

rx_status_t rx_quant_fp8(const void* const* srcs, int nsrc, size_t count,
                         rx_dtype_t src_dtype, rx_dtype_t fp8_dtype, int block,
                         void* const* codes, float* const* scales,
                         hipStream_t stream)
{
    if (!srcs || !codes || !scales)
        return RX_ERR_NULL;
    if (nsrc < 1 || nsrc > RX_MAX_SRC || !valid_block(block) || count > kMaxCount)
        return RX_ERR_ARG;
    if ((count / 256 + 1) * (size_t)nsrc >= ((size_t)1 << 32))   // 32-bit tile indices
        return RX_ERR_ARG;
    if (!hp_type(src_dtype) || !fp8_type(fp8_dtype))
        return RX_ERR_DTYPE;
    rx_status_t st = check_ptrs(srcs, nsrc, true);
    if (st != RX_OK)
        return st;
    st = check_ptrs(reinterpret_cast<const void* const*>(codes), nsrc, true);
    if (st != RX_OK)
        return st;
    st = check_ptrs(reinterpret_cast<const void* const*>(scales), nsrc, false);
    if (st != RX_OK)
        return st;
    if (count == 0)
        return RX_OK;
    rx::QuantArgs a = {};
    for (int j = 0; j < nsrc; ++j) {
        a.src[j] = srcs[j];
        a.codes[j] = codes[j];
        a.scales[j] = scales[j];
    }
    a.count = count;
    a.nsrc = nsrc;
    return launched(rx::launch_quant(a, src_dtype == RX_BF16 ? 1 : 0,
                                     fp8_dtype == RX_FP8_E5M2 ? 1 : 0, block, stream));
}

rx_status_t rx_dequant_reduce_requant(const void* const* codes,
                                      const float* const* scales, int nsrc,
                                      size_t count, rx_dtype_t fp8_dtype,
                                      int block, rx_drr_mode_t mode,
                                      void* out_codes, float* out_scales,
                                      void* out_hp, rx_dtype_t hp_dtype,
                                      hipStream_t stream)
{
    if (!codes || !scales)
        return RX_ERR_NULL;
    if (nsrc < 1 || nsrc > RX_MAX_SRC || !valid_block(block) || count > kMaxCount)
        return RX_ERR_ARG;
    if (mode != RX_DRR_SUM && mode != RX_DRR_REQUANT)
        return RX_ERR_ARG;
    const bool requant = mode == RX_DRR_REQUANT;
    if (requant) {
        if (!out_codes || !out_scales)
            return RX_ERR_NULL;
    } else {
        if (out_codes || out_scales)
            return RX_ERR_ARG;
        if (!out_hp)
            return RX_ERR_NULL;
    }
    if (!fp8_type(fp8_dtype) || (out_hp && !hp_type(hp_dtype)))
        return RX_ERR_DTYPE;
    rx_status_t st = check_ptrs(codes, nsrc, true);
    if (st != RX_OK)
        return st;
    st = check_ptrs(reinterpret_cast<const void* const*>(scales), nsrc, false);
    if (st != RX_OK)
        return st;
    if ((out_codes && !aligned16(out_codes)) || (out_scales && !aligned4(out_scales)) ||
        (out_hp && !aligned16(out_hp)))
        return RX_ERR_ALIGN;
    if (count == 0)
        return RX_OK;
    rx::DrrArgs a = {};
    for (int j = 0; j < nsrc; ++j) {
        a.codes[j] = codes[j];
        a.scales[j] = scales[j];
    }
    a.out_codes[0] = out_codes;
    a.out_scales[0] = out_scales;
    a.nout = requant ? 1 : 0;
    a.out_hp = out_hp;
    a.lo = 0;
    a.hi = count;
    a.block = block;
    a.hp_bf16 = hp_dtype == RX_BF16 ? 1 : 0;
    return launched(rx::launch_drr(a, nsrc, fp8_dtype == RX_FP8_E5M2 ? 1 : 0, requant, stream));
}

rx_status_t rx_lp_tree_chunk(size_t count, int nsrc, int block, int rank,
                             size_t* lo, size_t* hi)
{
    if (!lo || !hi)
        return RX_ERR_NULL;
    if (nsrc < 1 || nsrc > RX_MAX_SRC || rank < 0 || rank >= nsrc || !valid_block(block) ||
        count > kMaxCount)
        return RX_ERR_ARG;
    const size_t c = lp_chunk_len(count, nsrc, block);
    size_t a = (size_t)rank * c;
    if (a > count) a = count;
    size_t b = a + c;
    if (b > count) b = count;
    *lo = a;
    *hi = b;
    return RX_OK;
}

rx_status_t rx_lp_reduce_scatter_chunk_bcast(const void* const* codes,
                                             const float* const* scales, int nsrc,
                                             size_t count, rx_dtype_t fp8_dtype,
                                             int block, int rank,
                                             void* const* dst_codes,
                                             float* const* dst_scales,
                                             void* out_hp, rx_dtype_t hp_dtype,
                                             hipStream_t stream)
{
    if (!codes || !scales || !dst_codes || !dst_scales)
        return RX_ERR_NULL;
    if (nsrc < 1 || nsrc > RX_MAX_SRC || rank < 0 || rank >= nsrc || !valid_block(block) ||
        count > kMaxCount)
        return RX_ERR_ARG;
    if (!fp8_type(fp8_dtype) || (out_hp && !hp_type(hp_dtype)))
        return RX_ERR_DTYPE;
    rx_status_t st = check_ptrs(codes, nsrc, true);
    if (st == RX_OK)
        st = check_ptrs(reinterpret_cast<const void* const*>(scales), nsrc, false);
    if (st == RX_OK)
        st = check_ptrs(reinterpret_cast<const void* const*>(dst_codes), nsrc, true);
    if (st == RX_OK)
        st = check_ptrs(reinterpret_cast<const void* const*>(dst_scales), nsrc, false);
    if (st != RX_OK)
        return st;
    if (out_hp && !aligned16(out_hp))
        return RX_ERR_ALIGN;
    size_t lo = 0, hi = 0;
    rx_lp_tree_chunk(count, nsrc, block, rank, &lo, &hi);
    if (lo >= hi)
        return RX_OK;
    rx::DrrArgs a = {};
    for (int j = 0; j < nsrc; ++j) {
        a.codes[j] = codes[j];
        a.scales[j] = scales[j];
        a.out_codes[j] = dst_codes[j];
        a.out_scales[j] = dst_scales[j];
    }
    a.nout = nsrc;
    a.out_hp = out_hp;
    a.lo = lo;
    a.hi = hi;
    a.block = block;
    a.hp_bf16 = hp_dtype == RX_BF16 ? 1 : 0;
    return launched(rx::launch_drr(a, nsrc, fp8_dtype == RX_FP8_E5M2 ? 1 : 0, true, stream));
}

size_t rx_allreduce_local_workspace(int nsrc, size_t count, int block)
{
    if (nsrc < 1 || nsrc > RX_MAX_SRC || !valid_block(block) || count > kMaxCount)
        return 0;
    const size_t nb = (count + (size_t)block - 1) / (size_t)block;
    return (size_t)nsrc * (round256(count) + round256(nb * sizeof(float)));
}

rx_status_t rx_allreduce_local(void* const* bufs, int nsrc, size_t count,
                               rx_dtype_t dtype, rx_algo_t algo,
                               rx_dtype_t fp8_dtype, int block, void* workspace,
                               size_t workspace_bytes, hipStream_t stream)
{
    return allreduce_local_impl(bufs, nsrc, count, dtype, algo, fp8_dtype, block, workspace,
                                workspace_bytes, false, stream);
}

rx_status_t rx_allreduce_local_noalloc(void* const* bufs, int nsrc, size_t count,
                                       rx_dtype_t dtype, rx_algo_t algo,
                                       rx_dtype_t fp8_dtype, int block,
                                       hipStream_t stream)
{
    return allreduce_local_impl(bufs, nsrc, count, dtype, algo, fp8_dtype, block, nullptr,
                                RX_NOALLOC_SCRATCH_BYTES, true, stream);
}

}  // extern "C"
