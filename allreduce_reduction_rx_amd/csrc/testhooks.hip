// testhooks.hip -- kernels that run the device conversion and cross-lane
// helpers on their own, for exhaustive comparison with the CPU oracle.
#include <stdint.h>
#include <stdio.h>

#include "rx_device.hpp"
#include "rx_internal.hpp"
#include "rx_testhooks.h"

namespace rx {
namespace {

template <int F>
__global__ void k_enc_bits(uint32_t first, size_t n, uint8_t* out)
{
    const size_t i4 = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i4 >= n) return;
    float y[4];
    for (int k = 0; k < 4; ++k)
        y[k] = clamp_fmax<F>(bits_f32(first + (uint32_t)(i4 + k)));
    uint32_t w = f32x4_to_fp8<F>(y[0], y[1], y[2], y[3]);
    for (int k = 0; k < 4; ++k)
        if (i4 + k < n) out[i4 + k] = (uint8_t)(w >> (8 * k));
}

template <int F>
__global__ void k_dec(const uint8_t* in, size_t n, float* out)
{
    const size_t i4 = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i4 >= n) return;
    uint32_t w = 0;
    for (int k = 0; k < 4; ++k)
        if (i4 + k < n) w |= (uint32_t)in[i4 + k] << (8 * k);
    float d[4];
    fp8x4_to_f32<F>(w, d);
    for (int k = 0; k < 4; ++k)
        if (i4 + k < n) out[i4 + k] = d[k];
}

template <int F>
__global__ void k_scale_bits(uint32_t first, size_t n, float* s, float* r)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float sv, rv;
    block_scale<F>(bits_f32(first + (uint32_t)i), sv, rv);
    s[i] = sv;
    r[i] = rv;
}

__global__ void k_bf16_bits(uint32_t first, size_t n, uint16_t* out)
{
    const size_t i2 = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 2;
    if (i2 >= n) return;
    uint32_t p = pack_bf16(bits_f32(first + (uint32_t)i2), bits_f32(first + (uint32_t)(i2 + 1)));
    out[i2] = (uint16_t)(p & 0xFFFFu);
    if (i2 + 1 < n) out[i2 + 1] = (uint16_t)(p >> 16);
}

__global__ __launch_bounds__(64) void k_group_max(const uint32_t* in, int g, uint32_t* out)
{
    const size_t i = (size_t)blockIdx.x * 64 + threadIdx.x;
    out[i] = group_max_rt(in[i], g);
}

unsigned blocks_for(size_t threads) { return (unsigned)((threads + 255) / 256); }

}  // namespace
}  // namespace rx

namespace {

// Status of the launch just made: the triple-chevron launch reports through
// the per-thread last error, which each hook clears right before launching
// (it also holds whatever an earlier, unrelated HIP call returned).
rx_status_t launch_status()
{
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess)
        return RX_OK;
    fprintf(stderr, "librx: launch failed: %s\n", hipGetErrorName(e));
    return RX_ERR_HIP;
}

}  // namespace

extern "C" {

rx_status_t rxtest_fp8_encode_bits(uint32_t first, size_t n, rx_dtype_t fmt,
                                   uint8_t* out, hipStream_t stream)
{
    if (!out) return RX_ERR_NULL;
    if (fmt != RX_FP8_E4M3 && fmt != RX_FP8_E5M2) return RX_ERR_DTYPE;
    if (n > ((size_t)1 << 32) - first) return RX_ERR_ARG;
    if (n == 0) return RX_OK;
    const size_t th = (n + 3) / 4;
    (void)hipGetLastError();   // drop an earlier call's error
    if (fmt == RX_FP8_E4M3)
        hipLaunchKernelGGL(rx::k_enc_bits<rx::kE4M3>, dim3(rx::blocks_for(th)), dim3(256), 0, stream, first, n, out);
    else
        hipLaunchKernelGGL(rx::k_enc_bits<rx::kE5M2>, dim3(rx::blocks_for(th)), dim3(256), 0, stream, first, n, out);
    return launch_status();
}

rx_status_t rxtest_fp8_decode(const uint8_t* in, size_t n, rx_dtype_t fmt,
                              float* out, hipStream_t stream)
{
    if (!in || !out) return RX_ERR_NULL;
    if (fmt != RX_FP8_E4M3 && fmt != RX_FP8_E5M2) return RX_ERR_DTYPE;
    if (n == 0) return RX_OK;
    const size_t th = (n + 3) / 4;
    (void)hipGetLastError();   // drop an earlier call's error
    if (fmt == RX_FP8_E4M3)
        hipLaunchKernelGGL(rx::k_dec<rx::kE4M3>, dim3(rx::blocks_for(th)), dim3(256), 0, stream, in, n, out);
    else
        hipLaunchKernelGGL(rx::k_dec<rx::kE5M2>, dim3(rx::blocks_for(th)), dim3(256), 0, stream, in, n, out);
    return launch_status();
}

rx_status_t rxtest_block_scale_bits(uint32_t first, size_t n, rx_dtype_t fmt,
                                    float* s, float* r, hipStream_t stream)
{
    if (!s || !r) return RX_ERR_NULL;
    if (fmt != RX_FP8_E4M3 && fmt != RX_FP8_E5M2) return RX_ERR_DTYPE;
    if ((size_t)first + n > 0x80000000u) return RX_ERR_ARG;
    if (n == 0) return RX_OK;
    (void)hipGetLastError();   // drop an earlier call's error
    if (fmt == RX_FP8_E4M3)
        hipLaunchKernelGGL(rx::k_scale_bits<rx::kE4M3>, dim3(rx::blocks_for(n)), dim3(256), 0, stream, first, n, s, r);
    else
        hipLaunchKernelGGL(rx::k_scale_bits<rx::kE5M2>, dim3(rx::blocks_for(n)), dim3(256), 0, stream, first, n, s, r);
    return launch_status();
}

rx_status_t rxtest_bf16_round_bits(uint32_t first, size_t n, uint16_t* out, hipStream_t stream)
{
    if (!out) return RX_ERR_NULL;
    if (n > ((size_t)1 << 32) - first) return RX_ERR_ARG;
    if (n == 0) return RX_OK;
    const size_t th = (n + 1) / 2;
    (void)hipGetLastError();   // drop an earlier call's error
    hipLaunchKernelGGL(rx::k_bf16_bits, dim3(rx::blocks_for(th)), dim3(256), 0, stream, first, n, out);
    return launch_status();
}

rx_status_t rxtest_group_max(const uint32_t* in, size_t nwaves, int g, uint32_t* out,
                             hipStream_t stream)
{
    if (!in || !out) return RX_ERR_NULL;
    if (g < 1 || g > 64 || (g & (g - 1)) || nwaves > 0x7FFFFFFF) return RX_ERR_ARG;
    if (nwaves == 0) return RX_OK;
    (void)hipGetLastError();   // drop an earlier call's error
    hipLaunchKernelGGL(rx::k_group_max, dim3((unsigned)nwaves), dim3(64), 0, stream, in, g, out);
    return launch_status();
}

}  // extern "C"
