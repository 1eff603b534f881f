/*
 * rx_testhooks.h -- test entry points of librx that expose the device
 * conversion and cross-lane helpers the kernels are built from, so tests can
 * sweep them exhaustively against the CPU oracle. Same conventions as rx.h:
 * device pointers, asynchronous on `stream`, validation before any launch.
 */
#ifndef RX_TESTHOOKS_H
#define RX_TESTHOOKS_H

#include <stddef.h>
#include <stdint.h>
#include "rx.h"

#ifdef __cplusplus
extern "C" {
#endif

/* out[i] = OCP FP8 code of the FP32 pattern (first + i), after the kernels'
 * pre-clamp to [-FMAX, FMAX]; n <= 2^32 - first. fmt: RX_FP8_E4M3/E5M2.
 * NaN patterns give unspecified codes. out: n bytes. */
rx_status_t rxtest_fp8_encode_bits(uint32_t first, size_t n, rx_dtype_t fmt,
                                   uint8_t* out, hipStream_t stream);

/* out[i] = FP32 value of code in[i] (hardware decode). */
rx_status_t rxtest_fp8_decode(const uint8_t* in, size_t n, rx_dtype_t fmt,
                              float* out, hipStream_t stream);

/* out[i] = BF16 (round to nearest even) of the FP32 pattern (first + i). */
rx_status_t rxtest_bf16_round_bits(uint32_t first, size_t n, uint16_t* out,
                                   hipStream_t stream);

/* s[i], r[i] = the kernels' block scale and reciprocal for the block absmax
 * A = FP32 pattern (first + i): s = A / FMAX, r = FMAX / A (the correctly
 * rounded quotients), s = r = 1 for A == 0, s == 0 or r not finite (so also
 * for NaN); A = +inf gives s = +inf, r = 0. Patterns must have the sign bit
 * clear: first + n <= 0x80000000. */
rx_status_t rxtest_block_scale_bits(uint32_t first, size_t n, rx_dtype_t fmt,
                                    float* s, float* r, hipStream_t stream);

/* For each wave of 64 values in in[0 .. 64*nwaves): out[l] = max of in over
 * the aligned group of g lanes that holds lane l (g = 1, 2, 4, ..., 64),
 * computed with the kernels' DPP / permlane group maximum. */
rx_status_t rxtest_group_max(const uint32_t* in, size_t nwaves, int g,
                             uint32_t* out, hipStream_t stream);

/* Streaming ceiling kernels: the HBM rates that plain 16-byte-per-lane
 * streams reach on this GPU, measured beside the hot-path kernels.
 *   kind 0 (read):  reads `bytes` of src; every wave XORs what it read and
 *                   stores its 16-byte sum into dst[wave], so the XOR of dst
 *                   over rxtest_stream_sink_bytes(wgs_per_cu) bytes equals
 *                   the XOR of the 16-byte words of src.
 *   kind 1 (write): fills dst[0 .. bytes) with the FP32 pattern 1, 2, 3, 4
 *                   repeated; src is ignored (may be NULL).
 *   kind 2 (copy):  dst[0 .. bytes) = src[0 .. bytes).
 *   kind 3 (empty): the same launch with no memory access (the launch cost
 *                   alone); src, dst and bytes are ignored apart from the
 *                   alignment check, and it launches even for bytes == 0.
 * Launch: wgs_per_cu (1..8) workgroups of 256 threads per compute unit,
 * grid-stride over whole wave tiles of 4 vectors per lane, the partial last
 * tile after the loop; nontemporal != 0 uses
 * nontemporal loads and stores. bytes, src and dst must be multiples of 16
 * (RX_ERR_ALIGN); src and dst must not overlap. */
rx_status_t rxtest_stream(int kind, const void* src, void* dst, size_t bytes,
                          int wgs_per_cu, int nontemporal, hipStream_t stream);

/* Mixed read/write ceiling kernels: the access patterns of the hot-path
 * kernels with XOR in place of their arithmetic, so their rate is what the
 * memory system gives that mix of reads and writes.
 *   kind 0 (reduce): nsrc (1..16) sources of src_bytes each; dst (src_bytes)
 *                    = XOR of the sources, 16-byte word by word: nsrc : 1
 *                    bytes read : written (the flat reduce; nsrc = 1 copies).
 *   kind 1 (narrow 2:1), kind 2 (narrow 4:1): nsrc == 1; each 16-byte word
 *                    of the source is folded by XOR into 8 (kind 1: words
 *                    w0^w1, w2^w3) or 4 bytes (kind 2: w0^w1^w2^w3), written
 *                    at dst + 8 v or dst + 4 v: the quantizer's pattern for
 *                    BF16 (2:1) and FP32 (4:1) input.
 * srcs is a host array of device pointers (16-B aligned); src_bytes a
 * multiple of 16. Launch as rxtest_stream: wgs_per_cu (1..8) workgroups of
 * 256 threads per compute unit, grid-stride over wave tiles (reduce: 4
 * vectors per lane, 2 for more than 8 sources; narrow: 4, or 8 with the
 * prefetch), whole tiles in the loop and a partial last tile after it;
 * nontemporal != 0 uses nontemporal loads and stores; prefetch (0 or 1)
 * = 1 loads each wave's next tile into a second register buffer before it
 * writes the current one. dst must not overlap a source. */
rx_status_t rxtest_stream_mixed(int kind, const void* const* srcs, int nsrc, void* dst,
                                size_t src_bytes, int wgs_per_cu, int nontemporal, int prefetch,
                                hipStream_t stream);

/* The tree step's memory pattern without its arithmetic (a floor for it):
 * for j < n, bytes [offset_bytes, offset_bytes + bytes) of srcs[j] copied to
 * the same range of dsts[j] -- n read and n write streams, each its own
 * allocation. lanes 1: one lane per 16-byte vector (n loads, then n
 * stores); lanes 2: two lanes per vector, each copying half of the streams.
 * One thread per lane in workgroups of wg threads (64, 128 or 256), grid-
 * stride beyond 65536 workgroups; nontemporal loads and stores. srcs and
 * dsts are host arrays of device pointers (16-B aligned) whose buffers hold
 * at least offset_bytes + bytes; offset_bytes and bytes are multiples of 16;
 * a destination must not overlap a source. */
rx_status_t rxtest_copy_streams(const void* const* srcs, void* const* dsts, int n,
                                size_t offset_bytes, size_t bytes, int lanes, int wg,
                                hipStream_t stream);

/* Size in bytes of the read kernel's dst for this wgs_per_cu (0 if out of
 * range). */
size_t rxtest_stream_sink_bytes(int wgs_per_cu);

#ifdef __cplusplus
}
#endif
#endif /* RX_TESTHOOKS_H */
