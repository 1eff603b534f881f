/*
 * rx_oracle.h -- plain CPU oracle for the rx reduction library.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load, link or call this code. The
 * product path (the HIP library and its Python binding) never does, and it
 * shares no code, header, table or helper with this directory.
 *
 * Everything here is a slow, literal restatement of what the method
 * computes, in the order the definitions give, with no blocking or fusion:
 *
 *   - DDA flat: every rank reads all peers' buffers and reduces them locally
 *     (code-journey.com RCCLX article, "Core feature 1: Direct Data Access
 *     (DDA)", DDA Flat item), summing in FP32 ("Core feature 2: Low-Precision
 *     Collectives", feature table, row "Compute precision"), with SUM as the
 *     reduction ("Practical guide", usage example).
 *   - DDA tree: reduce-scatter then all-gather with direct access (same
 *     article, "Core feature 1", DDA Tree item); one rank's share is: reduce
 *     its chunk across all sources and write it into every destination.
 *   - Low-precision path: FP32/BF16 quantized to FP8, up to 4:1 ("Core
 *     feature 2", opening paragraph and table row "Data types"), reduced in
 *     FP32 after dequantization.
 *
 * Where the pages are silent, the readings taken are:
 *   - FP8 formats are OCP E4M3 (E4M3FN, max 448) and E5M2 (max 57344);
 *     encode rounds to nearest, ties to even, and saturates to +-max.
 *   - Each block of B consecutive elements carries one FP32 scale
 *     s = A / FMAX (A = block absmax); elements are multiplied by
 *     r = FMAX / A (each a single correctly rounded FP32 division) and then
 *     encoded.  A == 0, s == 0 or r not finite gives s = r = 1.
 *   - Sums fold left in source order 0..N-1, starting from source 0, each
 *     addition rounded to FP32; dequantization is fl32(decode(c) * s), never
 *     fused with the addition.
 *   - Requantization reuses the input block size and format; its optional
 *     high-precision output is dequant(requant(S)), the value every rank
 *     would see after the all-gather.
 *   - Tree chunks: c = roundup(ceil(count / N), 16 / elem_size);
 *     chunk k = [min(k c, count), min(k c + c, count)).
 *
 * All functions are single-threaded and pure (no global state).
 */
#ifndef RX_ORACLE_H
#define RX_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. Values match the library's dtype enum only by convention;
 * nothing here includes the library's header. */
enum { RXO_FP32 = 0, RXO_BF16 = 1, RXO_E4M3 = 2, RXO_E5M2 = 3 };
enum { RXO_DRR_SUM = 0, RXO_DRR_REQUANT = 1 };

/* ---- scalar codecs ---------------------------------------------------- */
float    rxo_bf16_to_f32(uint16_t h);           /* exact widening          */
uint16_t rxo_f32_to_bf16(float x);              /* round to nearest even   */
float    rxo_fp8_max(int fmt);                  /* 448 or 57344            */
float    rxo_fp8_decode(uint8_t code, int fmt); /* exact value of a code   */
uint8_t  rxo_fp8_encode(float v, int fmt);      /* RNE, saturating         */

/* Array forms of the codecs (test helpers; element i of out from in[i]). */
void rxo_fp8_encode_array(const float* in, size_t n, int fmt, uint8_t* out);
void rxo_fp8_encode_bits_range(uint32_t first, uint32_t n, int fmt, uint8_t* out);
void rxo_f32_to_bf16_array(const float* in, size_t n, uint16_t* out);
void rxo_fp8_decode_array(const uint8_t* in, size_t n, int fmt, float* out);

/* ---- block scale ------------------------------------------------------ */
/* Scale and reciprocal of one block of FP32 values (already widened). */
void rxo_block_scale(const float* x, size_t len, int fmt, float* s, float* r);
/* Test helper: s[i], r[i] of the one-element block {A}, A = FP32 pattern
 * (first + i). */
void rxo_block_scale_bits_range(uint32_t first, uint32_t n, int fmt, float* s, float* r);

/* ---- hot-path operations ---------------------------------------------- */
/* y[i] = cast(fold_r x_r[i]); dtype FP32 or BF16 for sources and dst. */
void rxo_reduce_flat(const void* const* srcs, int nsrc, size_t count,
                     int dtype, void* dst);

/* Chunk bounds [lo, hi) owned by `rank` in the tree step. */
void rxo_tree_chunk(size_t count, int nsrc, int dtype, int rank,
                    size_t* lo, size_t* hi);

/* Reduce chunk `rank` across the sources, write it into every dsts[j]. */
void rxo_reduce_scatter_chunk_bcast(const void* const* srcs, int nsrc,
                                    size_t count, int dtype, int rank,
                                    void* const* dsts);

/* Quantize each source: codes[j][i] (uint8), scales[j][b] (FP32). */
void rxo_quant_fp8(const void* const* srcs, int nsrc, size_t count,
                   int src_dtype, int fmt, int block,
                   uint8_t* const* codes, float* const* scales);

/* Dequantize every source, fold in FP32; SUM mode writes the sum to out_hp
 * (FP32 or BF16); REQUANT mode writes out_codes/out_scales and, when out_hp
 * is not NULL, dequant(requant(sum)) cast to hp_dtype. */
void rxo_dequant_reduce_requant(const uint8_t* const* codes,
                                const float* const* scales, int nsrc,
                                size_t count, int fmt, int block, int mode,
                                uint8_t* out_codes, float* out_scales,
                                void* out_hp, int hp_dtype);

/* Low-precision tree step (one rank's share of a low-precision
 * reduce-scatter + all-gather). Chunks are whole scale blocks:
 * c = roundup(ceil(count / nsrc), block); chunk k = [min(k c, count),
 * min(k c + c, count)). */
void rxo_lp_tree_chunk(size_t count, int nsrc, int block, int rank,
                       size_t* lo, size_t* hi);

/* Dequantize + FP32 sum + requantize the blocks of chunk `rank`, and write
 * the requantized codes and scales of the chunk into every dst_codes[j] /
 * dst_scales[j] (message-indexed; nothing outside the chunk is written).
 * When out_hp is not NULL, its chunk receives dequant(requant(sum)). */
void rxo_lp_reduce_scatter_chunk_bcast(const uint8_t* const* codes,
                                       const float* const* scales, int nsrc,
                                       size_t count, int fmt, int block,
                                       int rank, uint8_t* const* dst_codes,
                                       float* const* dst_scales,
                                       void* out_hp, int hp_dtype);

/* Whole allreduce of nsrc rank buffers on one GPU, in place: afterwards
 * every bufs[j] holds the result. algo 1 (flat) and 2 (tree) give the FP32
 * left fold cast to dtype; algo 3 (low precision) gives, for every rank,
 * the dequantization of the requantized FP32 sum of the quantized inputs
 * (quantize each rank, reduce-scatter + all-gather of the FP8 chunks,
 * dequantize). */
enum { RXO_ALGO_FLAT = 1, RXO_ALGO_TREE = 2, RXO_ALGO_LOWPREC = 3 };
void rxo_allreduce_local(void* const* bufs, int nsrc, size_t count, int dtype,
                         int algo, int fmt, int block);

#ifdef __cplusplus
}
#endif
#endif /* RX_ORACLE_H */
