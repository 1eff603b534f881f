// rx_device.hpp -- gfx950 device helpers shared by the rx kernels:
// 16-byte vector memory access, BF16/FP8 conversions on the hardware
// converters, and cross-lane maxima on DPP / permlane swaps.
//
// Everything here is written for CDNA4 (gfx950), wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rx {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// FP8 formats (OCP). E4M3 = E4M3FN: largest finite 448; E5M2: 57344.
enum Fp8 { kE4M3 = 0, kE5M2 = 1 };

template <int F> struct Fp8Traits;
template <> struct Fp8Traits<kE4M3> { static constexpr float kMax = 448.0f; };
template <> struct Fp8Traits<kE5M2> { static constexpr float kMax = 57344.0f; };

// ---------------------------------------------------------------------------
// Memory
// ---------------------------------------------------------------------------

__device__ __forceinline__ u32x4 ld16(const void* base, size_t vec)
{
    return reinterpret_cast<const u32x4*>(base)[vec];
}

// Streaming load: data read once, not worth keeping in the caches.
__device__ __forceinline__ u32x4 ld16_stream(const void* base, size_t vec)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + vec);
}

__device__ __forceinline__ void st16(void* base, size_t vec, u32x4 v)
{
    reinterpret_cast<u32x4*>(base)[vec] = v;
}

__device__ __forceinline__ void st16_stream(void* base, size_t vec, u32x4 v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(base) + vec);
}

// ---------------------------------------------------------------------------
// BF16 <-> FP32
// ---------------------------------------------------------------------------

// The two BF16 halves of a dword, widened exactly to FP32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Two FP32 -> packed BF16 pair (lo in bits 0..15), round to nearest even on
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    f32x2 v = {lo, hi};
    bf16x2 b = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

// ---------------------------------------------------------------------------
// FP8 (OCP) on the gfx950 converters
// ---------------------------------------------------------------------------

// Four codes of a dword -> FP32 (byte k -> out[k]); exact.
template <int F>
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* out)
{
    f32x2 a, b;
    if constexpr (F == kE4M3) {
        a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
        b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    } else {
        a = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
        b = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true);
    }
    out[0] = a[0]; out[1] = a[1]; out[2] = b[0]; out[3] = b[1];
}

// Four FP32 values, already inside [-FMAX, FMAX], -> four codes (x[k] -> byte
// k), round to nearest even. Pre-clamping makes the conversion saturating.
template <int F>
__device__ __forceinline__ uint32_t f32x4_to_fp8(float x0, float x1, float x2, float x3)
{
    int w;
    if constexpr (F == kE4M3) {
        w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
    } else {
        w = __builtin_amdgcn_cvt_pk_bf8_f32(x0, x1, 0, false);
        w = __builtin_amdgcn_cvt_pk_bf8_f32(x2, x3, w, true);
    }
    return (uint32_t)w;
}

template <int F>
__device__ __forceinline__ float clamp_fmax(float y)
{
    constexpr float m = Fp8Traits<F>::kMax;
    return __builtin_amdgcn_fmed3f(y, -m, m);
}

// Block scale and its reciprocal from the block absmax A: s = A / FMAX and
// r = FMAX / A, each the correctly rounded FP32 quotient; A == 0, s == 0 or
// r not finite gives s = r = 1.
//
// Both quotients are FMA-corrected products (P. Markstein, "IA-64 and
// Elementary Functions", Prentice Hall 2000: for a quotient b / d with an
// approximation y of 1 / d, q0 = b y, e = b - q0 d, exact with an FMA, and
// q = q0 + e y): 10 instructions instead of two division sequences of 11.
// s takes y = RN(1 / FMAX), a compile-time constant. r takes the hardware
// reciprocal of A / 4, refined by one Newton step, and divides FMAX / 4 by
// A / 4: the quarter scaling is exact wherever the result is not degenerate
// and keeps the reciprocal normal up to A = FLT_MAX. Checked against IEEE
// division for every finite A >= 0 with every reciprocal estimate within
// 1 ulp of the true one (tests/bruteforce/block_scale_sweep.c), and on the
// GPU against the oracle for every A up to +inf.
template <int F>
__device__ __forceinline__ void block_scale(float a, float& s, float& r)
{
    constexpr float m = Fp8Traits<F>::kMax;
    constexpr float inv_m = 1.0f / m;      // RN(1 / FMAX)
    constexpr float m4 = 0.25f * m;
    const float q0 = a * inv_m;
    float sv = __builtin_fmaf(__builtin_fmaf(-q0, m, a), inv_m, q0);
    const float a4 = 0.25f * a;
    const float y0 = __builtin_amdgcn_rcpf(a4);
    const float y1 = __builtin_fmaf(__builtin_fmaf(-a4, y0, 1.0f), y0, y0);
    const float p0 = m4 * y1;
    float rv = __builtin_fmaf(__builtin_fmaf(-p0, a4, m4), y1, p0);
    // A = +inf: the quotients are +inf and 0 (the sequences give NaN)
    const bool inf = a == __builtin_inff();
    sv = inf ? a : sv;
    rv = inf ? 0.0f : rv;
    bool degenerate = (a == 0.0f) | (sv == 0.0f) | !__builtin_isfinite(rv);
    s = degenerate ? 1.0f : sv;
    r = degenerate ? 1.0f : rv;
}

// ---------------------------------------------------------------------------
// Cross-lane maximum over aligned groups of G lanes (G = 1..64, power of 2).
// Operates on |x| bit patterns: for non-NaN values the unsigned order of the
// magnitude bits is the order of the magnitudes, and max is exact.
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

template <int Ctrl>
__device__ __forceinline__ uint32_t dpp(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, Ctrl, 0xF, 0xF, false);
}

template <int G>
__device__ __forceinline__ uint32_t group_max(uint32_t v)
{
    static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "group size");
    if constexpr (G >= 2) v = umax(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
    if constexpr (G >= 4) v = umax(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
    if constexpr (G >= 8) v = umax(v, dpp<0x141>(v));  // row_half_mirror
    if constexpr (G >= 16) v = umax(v, dpp<0x140>(v)); // row_mirror
    if constexpr (G >= 32) {                           // rows 0<->1, 2<->3
        auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        v = umax(p[0], p[1]);
    }
    if constexpr (G >= 64) {                           // halves 0<->1
        auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        v = umax(p[0], p[1]);
    }
    return v;
}

// Runtime group size (wave-uniform), for kernels whose block size is an
// argument.
__device__ __forceinline__ uint32_t group_max_rt(uint32_t v, int g)
{
    if (g >= 2) v = umax(v, dpp<0xB1>(v));
    if (g >= 4) v = umax(v, dpp<0x4E>(v));
    if (g >= 8) v = umax(v, dpp<0x141>(v));
    if (g >= 16) v = umax(v, dpp<0x140>(v));
    if (g >= 32) {
        auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        v = umax(p[0], p[1]);
    }
    if (g >= 64) {
        auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        v = umax(p[0], p[1]);
    }
    return v;
}

__device__ __forceinline__ uint32_t abs_bits(float x) { return __builtin_bit_cast(uint32_t, x) & 0x7FFFFFFFu; }
__device__ __forceinline__ float bits_f32(uint32_t u) { return __builtin_bit_cast(float, u); }

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// MI355X dispatches workgroup b to XCD b % 8, and each XCD has its own L2.
// Renumber workgroups so that each XCD owns one contiguous range of the g
// workgroup ids (a bijection on [0, g)); data shared by neighbouring tiles
// (a cache line of block scales) is then fetched once per XCD range instead
// of once per XCD.
constexpr uint32_t kXcds = 8;

// XCD x owns q + 1 ids from x (q + 1) if x < r, else q ids from
// r (q + 1) + (x - r) q; both starts equal x q + min(x, r). Written without a
// branch, so a kernel's scalar loads are not held behind one.
__host__ __device__ constexpr uint32_t xcd_contiguous(uint32_t b, uint32_t g)
{
    const uint32_t q = g / kXcds, r = g % kXcds, x = b % kXcds, i = b / kXcds;
    return x * q + (x < r ? x : r) + i;
}

// Nonzero iff p is not null. A kernel that tests its pointers for null in
// the same condition as its range check has them loaded before that branch,
// together with the other kernel arguments, instead of after it (one scalar
// round trip less before its first global load).
__device__ __forceinline__ uint32_t ptr_nonzero(const void* p)
{
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    return (uint32_t)v | (uint32_t)(v >> 32);
}

}  // namespace rx
