// drr.hip -- launch of the dequantize-reduce-requantize kernel (drr.hpp):
// lane layout and launch geometry by message size and output type.
#include <stdio.h>

#include "drr.hpp"

namespace rx {
namespace {

// One wave per tile (64 threads per work item). Large messages: 256-thread
// workgroups, at most 2 per CU (a narrow HBM access window measured best on
// MI355X), also for the one-source FP32-output layout (4 x 4: 16M codes
// E5M2/256 15.8 us against 16.0 us with 4 per CU, 256M codes 232 against
// more than 249 us); decode-size messages: one tile per wave over every CU.
LaunchPolicy policy_drr() { return {64u, 256u, 2u}; }
LaunchPolicy policy_drr_fp32_out() { return {64u, 256u, 2u}; }
// One source (the separate dequantization): each wave reads 1/N of the bytes
// of an N-source launch, so more waves keep HBM busy; 4 workgroups per CU
// measured 14% faster than 2 at 8 x 512 MiB BF16 (6 and 8 slower again).
LaunchPolicy policy_drr_one_source() { return {64u, 256u, 4u}; }

// The range [lo, hi) of a as a range that starts at code 0: every pointer
// offset to code lo (a block multiple), lo = 0, hi = hi - lo.
DrrArgs from_lo(const DrrArgs& a, int nsrc)
{
    DrrArgs arg = a;
    const size_t esz = a.hp_bf16 ? 2 : 4;
    const size_t blk0 = a.lo / (size_t)a.block;
    for (int j = 0; j < nsrc; ++j) {
        arg.codes[j] = static_cast<const uint8_t*>(a.codes[j]) + a.lo;
        arg.scales[j] = a.scales[j] + blk0;
    }
    for (int j = 0; j < kMaxSrc; ++j) {
        if (a.out_codes[j]) arg.out_codes[j] = static_cast<uint8_t*>(a.out_codes[j]) + a.lo;
        if (a.out_scales[j]) arg.out_scales[j] = a.out_scales[j] + blk0;
        if (a.out_hps[j]) arg.out_hps[j] = static_cast<uint8_t*>(a.out_hps[j]) + a.lo * esz;
    }
    if (a.out_hp) arg.out_hp = static_cast<uint8_t*>(a.out_hp) + a.lo * esz;
    arg.lo = 0;
    arg.hi = a.hi - a.lo;
    return arg;
}

// Codes [a.lo + done, a.hi) -- less than one tile -- in k_drr (fns' layout),
// one 64-thread workgroup; nothing when done covers the range. done is a
// multiple of the tile, so of the block.
hipError_t launch_rest(const DrrArgs& a, int nsrc, int fmt, int r, size_t done, const DrrFns& fns, hipStream_t s)
{
    if (a.lo + done >= a.hi)
        return hipSuccess;
    DrrArgs arg = a;
    arg.lo = a.lo + done;
    arg.xcd_ranges = 0;
    void* params[] = {&arg};
    return launch_logged("k_drr (ragged remainder)", (const void*)fns.fn[fmt][r][nsrc - 1], dim3(1), dim3(kWave),
                         params, s);
}

}  // namespace

hipError_t launch_drr(const DrrArgs& a, int nsrc, int fmt, bool requant, hipStream_t s)
{
    const size_t cus = (size_t)device_cu_count();
    const size_t len = a.hi - a.lo;
    const bool small = (len + 1023) / 1024 < kSmallTilesPerCu * cus / 2;
    const bool all = requant && a.out_hps[0] != nullptr;   // every rank's buffer
    const bool fp32_out = (a.out_hp != nullptr || all) && !a.hp_bf16;
    const bool codes_only = requant && !all && a.out_hp == nullptr;
    // chunk layout (codes per lane per chunk, chunks per lane); block / CPC <= 64
    int cpc = 16, u = 1;
    bool staged = false;
    const bool hp_out = a.out_hp != nullptr || all;
    if (small) {
        if (a.block <= 256) cpc = 4;
    } else if (hp_out && nsrc >= 2) {
        // FP32 or BF16 output from several sources: 16 codes per lane
        // (16-byte code loads) with the output staged through LDS into
        // contiguous 1 KiB stores. 8 x 16M codes E4M3/128 with FP32 output:
        // 42.1 -> 37.8 us against 4 x 4; 8 x 64M codes E5M2/256 with BF16
        // output: 127.5 -> 120.6 us against 8 x 2
        staged = true;
    } else if (fp32_out) {
        // one source (the separate dequantization): 4 x 4 measured the same
        // as staging
        if (a.block <= 256) { cpc = 4; u = 4; }
    } else if (a.block <= 512 && !codes_only) {
        // BF16 output from one source; codes only (one destination or a
        // push to N) keep 16 x 1: 16-byte code stores measured 7-13% faster
        // at 8 x 4M..64M codes with one destination and 1-3% with N
        cpc = 8;
        u = 2;
    }
    const size_t tile = (size_t)kWave * cpc * u;
    const size_t tiles = (len + tile - 1) / tile;
    const int r = !requant ? kDrrSum : all ? kDrrRequantAll : a.nout > 1 ? kDrrRequantPush : kDrrRequant;
    if (staged) {
        // Whole tiles of 1024 codes in the staged kernel, two 256-thread
        // workgroups per CU, each XCD a contiguous range up to 128 tiles per
        // CU with FP32 output and 512 with BF16 output, plain order above
        // (FP32: 8 x 16M codes 37.8 against 39.1 us, 8 x 64M 146 against
        // 152 us; BF16: 8 x 64M 119.8 against 122.1 us, 8 x 256M 513
        // against 524 us); a ragged remainder (less than one tile) in the
        // unstaged 16 x 1 kernel, launched after it.
        // Requantization from 256 tiles per CU: the prefetching
        // k_drr_staged_pf at one workgroup per CU in plain order (8 x 256M
        // codes E5M2/256 with BF16 output 502.1 -> 481.4 us, 8 x 64M with FP32
        // output 144.8 -> 143.3 us; at 8 x 16M, 64 tiles per CU, it was 1.7%
        // slower).
        const size_t whole = len / tile;
        if (whole) {
            const bool pf = r == kDrrRequant && whole >= (size_t)256 * cus;
            LaunchPolicy pol = policy_drr();
            if (pf)
                pol.max_wgs_per_cu = 1;
            dim3 grid, blk;
            launch_geometry(whole * kWave, false, pol, grid, blk);
            DrrArgs arg = from_lo(a, nsrc);
            arg.hi = whole * tile;
            arg.xcd_ranges = !pf && whole <= (size_t)(a.hp_bf16 ? 512 : 128) * cus ? 1 : 0;
            void* params[] = {&arg};
            const DrrFn fn = pf ? drr_fns_pf().staged[a.hp_bf16 ? 1 : 0][fmt][nsrc - 1]
                                : drr_fns_16x1_staged(a.hp_bf16).fn[fmt][r][nsrc - 1];
            const hipError_t e = launch_logged(pf ? "k_drr_staged_pf" : "k_drr_staged", (const void*)fn, grid, blk,
                                               params, s);
            if (e != hipSuccess)
                return e;
        }
        return launch_rest(a, nsrc, fmt, r, whole * tile, drr_fns_16x1(), s);
    }
    LaunchPolicy pol = (cpc == 4 && u == 4) ? policy_drr_fp32_out()
                     : nsrc == 1            ? policy_drr_one_source()
                                            : policy_drr();
    // Medium messages with one requantized output: when two workgroups per
    // CU would give each wave fewer than 16 tiles, four per CU in
    // XCD-contiguous order balance the end of the launch (8 x 16M codes
    // E4M3/128: 30.2 -> 27.9 us; 8 x 256M codes: two per CU stay best).
    const bool medium = !small && r == kDrrRequant && cpc == 8 &&
                        tiles < (size_t)16 * 2 * (256 / kWave) * cus;
    if (medium)
        pol.max_wgs_per_cu = 4;
    // Codes only, one destination (16 x 1): below 32 tiles per CU four
    // workgroups per CU in plain order; up to 512 per CU, two per CU with
    // each XCD a contiguous range; above, two per CU in plain order (8 x 4M
    // codes E4M3/128: 7.1 us against 8.2 us with two per CU; 8 x 16M:
    // 25.4 us, 8 x 64M: 100.7 us against 105.1 us in plain order; 8 x 256M
    // E5M2/256: 431.5 us against 437.7 us XCD-contiguous).
    const bool single_codes = !small && r == kDrrRequant && cpc == 16 && codes_only;
    const bool few = single_codes && tiles < (size_t)32 * cus;
    const bool many = single_codes && tiles > (size_t)512 * cus;
    if (few)
        pol.max_wgs_per_cu = 4;
    dim3 grid, blk;
    launch_geometry(tiles * kWave, small, pol, grid, blk);
    DrrArgs arg = a;
    // Give each XCD a contiguous range of tiles, so that the tiles sharing a
    // 128-byte line of block scales (loaded, and written to every
    // destination) meet in one L2. Measured: decode-size 8% faster; large
    // pushes to N destinations 3-8% and the FP32-output layout 2% faster;
    // no gain for the other large layouts, which keep the plain order.
    arg.xcd_ranges = (small || medium || r == kDrrRequantPush || (cpc == 4 && u == 4) ||
                      (single_codes && !few && !many)) ? 1 : 0;
    if (small && blk.x == (unsigned)kWave) {
        // Decode-size launches (one tile per 64-thread workgroup): each XCD
        // takes a contiguous range of tiles that covers whole 128-byte lines
        // of block scales (32 blocks), so that no line of scales is written
        // in part by one XCD and in part by another. 8 x 32K-code chunks
        // pushed to 8 destinations (E5M2/256, 128 tiles: 4 XCDs x 32):
        // 2.64 -> 2.48 us, FETCH_SIZE 170 -> 157 KiB.
        const size_t tiles_per_line = (size_t)32 * (size_t)a.block / tile > 0
                                      ? (size_t)32 * (size_t)a.block / tile : 1;
        const size_t lines = (tiles + tiles_per_line - 1) / tiles_per_line;
        const size_t range = (lines + kXcds - 1) / kXcds * tiles_per_line;
        arg.xcd_ranges = (int)range;
        grid = dim3((unsigned)(kXcds * range));
        if (cpc == 4 && len % tile == 0) {
            // a range of whole tiles: the loop-free kernel
            void* params[] = {&arg};
            return launch_logged("k_drr_tile1 (decode size)", (const void*)drr_fns_4x1_tile1().fn[fmt][r][nsrc - 1],
                                 grid, blk, params, s);
        }
    }
    if (!small && cpc == 16) {
        // 16 x 1: whole tiles in k_drr_whole (no partial-tile path in its
        // loop), then the ragged remainder (less than one tile) in k_drr.
        // Codes only to one destination from 512 tiles per CU: the
        // prefetching k_drr_pf at one workgroup per CU, XCD-contiguous
        // (8 x 128M codes E5M2/256: 207.7 -> 204.6 us; 8 x 256M: 441.8 ->
        // 425.4 us; at 8 x 16M it was 3% slower than k_drr_whole).
        const bool pf = single_codes && tiles >= (size_t)512 * cus;
        const size_t whole = len / tile;
        if (whole) {
            DrrArgs warg = from_lo(a, nsrc);
            warg.hi = whole * tile;
            warg.xcd_ranges = pf ? 1 : arg.xcd_ranges;
            LaunchPolicy wpol = pol;
            if (pf)
                wpol.max_wgs_per_cu = 1;
            launch_geometry(whole * kWave, false, wpol, grid, blk);
            void* params[] = {&warg};
            const DrrFn wfn = pf ? drr_fns_pf().codes16[fmt][nsrc - 1] : drr_fns_16x1_whole().fn[fmt][r][nsrc - 1];
            const hipError_t e = launch_logged(pf ? "k_drr_pf" : "k_drr_whole", (const void*)wfn, grid, blk, params, s);
            if (e != hipSuccess)
                return e;
        }
        return launch_rest(a, nsrc, fmt, r, whole * tile, drr_fns_16x1(), s);
    }
    if (!small && r == kDrrSum && nsrc == 1 && ((cpc == 4 && u == 4) || (cpc == 8 && u == 2))) {
        // The one-source dequantization in 4 x 4 (FP32) or 8 x 2 (BF16):
        // whole tiles in the prefetching k_drr_pf at two workgroups per CU,
        // XCD-contiguous (16M codes E4M3/128 to FP32: 16.36 -> 15.66 us, 64M:
        // 59.2 -> 57.7 us; 64M codes E5M2/256 to BF16: 36.2 -> 35.0 us,
        // 256M: 140.6 -> 139.6 us), then the ragged remainder in k_drr. As
        // whole-tile kernels without the prefetch these layouts measured
        // slower than k_drr (16M codes to FP32 16.4 -> 17.3 us).
        const size_t whole = len / tile;
        if (whole) {
            DrrArgs warg = from_lo(a, nsrc);
            warg.hi = whole * tile;
            warg.xcd_ranges = 1;
            LaunchPolicy wpol = pol;
            wpol.max_wgs_per_cu = 2;
            launch_geometry(whole * kWave, false, wpol, grid, blk);
            void* params[] = {&warg};
            const DrrFn wfn = cpc == 4 ? drr_fns_pf().sum44[fmt] : drr_fns_pf().sum82[fmt];
            const hipError_t e = launch_logged("k_drr_pf (one source)", (const void*)wfn, grid, blk, params, s);
            if (e != hipSuccess)
                return e;
        }
        return launch_rest(a, nsrc, fmt, r, whole * tile, cpc == 4 ? drr_fns_4x4() : drr_fns_8x2(), s);
    }
    void* params[] = {&arg};
    const DrrFn fn = cpc == 4 ? (u == 4 ? drr_fns_4x4().fn[fmt][r][nsrc - 1] : drr_fns_4x1().fn[fmt][r][nsrc - 1])
                   : cpc == 8 ? drr_fns_8x2().fn[fmt][r][nsrc - 1] : drr_fns_16x1().fn[fmt][r][nsrc - 1];
    char what[64] = "k_drr";
    if (debug_enabled())
        snprintf(what, sizeof what, "k_drr mode %d layout %dx%d", r, cpc, u);
    return launch_logged(what, (const void*)fn, grid, blk, params, s);
}

}  // namespace rx
