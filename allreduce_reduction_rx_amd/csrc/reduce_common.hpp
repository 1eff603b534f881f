// reduce_common.hpp -- helpers of the DDA flat reduce and the DDA tree step
// (reduce.hip, tree.hip): N-source 16-byte folds in FP32 and element-wise
// tails.
#pragma once

#include <array>
#include <utility>

#include "rx_device.hpp"
#include "rx_internal.hpp"

namespace rx {
namespace {

template <int DT> struct Elem;
template <> struct Elem<0> { static constexpr int kVE = 4; };  // FP32: 4 per 16 B
template <> struct Elem<1> { static constexpr int kVE = 8; };  // BF16: 8 per 16 B

// Fold vector `v` (16 bytes) of N sources; returns the narrowed 16 bytes.
// NT: nontemporal source loads (data read once). Every element is summed in
// source order 0..N-1 in both loop orders: SM (source-major) adds each
// source into all the elements as its load arrives, otherwise one element's
// sum is completed at a time. The order only changes the instruction
// schedule; measured on MI355X, source-major is faster for the tree step
// (8 x 4 MiB BF16: 2.94 against 3.05 us) and element-major for the
// decode-size flat reduce (8 x 512 KiB: 2.68 against 2.83 us).
template <int DT, int N, bool NT, bool SM = false>
__device__ __forceinline__ u32x4 fold_vec(const void* const* src, size_t v)
{
    u32x4 x[N];
#pragma unroll
    for (int r = 0; r < N; ++r)
        x[r] = NT ? ld16_stream(src[r], v) : ld16(src[r], v);
    constexpr int VE = Elem<DT>::kVE;
    float acc[VE];
    u32x4 out;
    if constexpr (SM) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if constexpr (DT == 0) {
                acc[k] = bits_f32(x[0][k]);
            } else {
                acc[2 * k] = bf16_lo(x[0][k]);
                acc[2 * k + 1] = bf16_hi(x[0][k]);
            }
        }
#pragma unroll
        for (int r = 1; r < N; ++r) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if constexpr (DT == 0) {
                    acc[k] = acc[k] + bits_f32(x[r][k]);
                } else {
                    acc[2 * k] = acc[2 * k] + bf16_lo(x[r][k]);
                    acc[2 * k + 1] = acc[2 * k + 1] + bf16_hi(x[r][k]);
                }
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k)
            out[k] = DT == 0 ? __builtin_bit_cast(uint32_t, acc[k]) : pack_bf16(acc[2 * k], acc[2 * k + 1]);
    } else if constexpr (DT == 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float a = bits_f32(x[0][k]);
#pragma unroll
            for (int r = 1; r < N; ++r)
                a = a + bits_f32(x[r][k]);
            out[k] = __builtin_bit_cast(uint32_t, a);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float lo = bf16_lo(x[0][k]);
            float hi = bf16_hi(x[0][k]);
#pragma unroll
            for (int r = 1; r < N; ++r) {
                lo = lo + bf16_lo(x[r][k]);
                hi = hi + bf16_hi(x[r][k]);
            }
            out[k] = pack_bf16(lo, hi);
        }
    }
    return out;
}

// Fold 16-byte vectors already loaded (x[r] from source r), in source order
// 0..N-1 per element; returns the narrowed 16 bytes.
template <int DT, int N>
__device__ __forceinline__ u32x4 fold_regs(const u32x4 (&x)[N])
{
    u32x4 out;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if constexpr (DT == 0) {
            float acc = bits_f32(x[0][k]);
#pragma unroll
            for (int r = 1; r < N; ++r)
                acc = acc + bits_f32(x[r][k]);
            out[k] = __builtin_bit_cast(uint32_t, acc);
        } else {
            float lo = bf16_lo(x[0][k]);
            float hi = bf16_hi(x[0][k]);
#pragma unroll
            for (int r = 1; r < N; ++r) {
                lo = lo + bf16_lo(x[r][k]);
                hi = hi + bf16_hi(x[r][k]);
            }
            out[k] = pack_bf16(lo, hi);
        }
    }
    return out;
}

// One element i (tail of a count that is not a multiple of 16 bytes).
template <int DT, int N>
__device__ __forceinline__ float fold_vec_tail(const void* const* src, size_t i)
{
    float acc;
    if constexpr (DT == 0) {
        acc = static_cast<const float*>(src[0])[i];
#pragma unroll
        for (int r = 1; r < N; ++r)
            acc = acc + static_cast<const float*>(src[r])[i];
    } else {
        acc = bits_f32((uint32_t)static_cast<const uint16_t*>(src[0])[i] << 16);
#pragma unroll
        for (int r = 1; r < N; ++r)
            acc = acc + bits_f32((uint32_t)static_cast<const uint16_t*>(src[r])[i] << 16);
    }
    return acc;
}

template <int DT>
__device__ __forceinline__ void store_elem(void* dst, size_t i, float v)
{
    if constexpr (DT == 0)
        static_cast<float*>(dst)[i] = v;
    else
        static_cast<uint16_t*>(dst)[i] = (uint16_t)(pack_bf16(v, 0.0f) & 0xFFFFu);
}

// Jobs below this many 16-byte vectors per CU run the decode-size kernels.
inline bool small_job(size_t threads) { return threads < kSmallThreadsPerCu * (size_t)device_cu_count(); }

}  // namespace
}  // namespace rx
