/*
 * rx.h -- C ABI of librx, the one-GPU data-parallel core of the RCCLX
 * allreduce paths, written for AMD Instinct MI355X (gfx950).
 *
 * The pages this library follows describe Meta's RCCLX (the RCCLX article on
 * code-journey.com, pt and ko editions, and its Chinese summary on
 * ai-stack.site). On one GPU, the N "rank" buffers of a collective are N
 * separate device allocations; every entry point takes an array of those
 * pointers and performs one rank's local share of the collective.
 *
 * Conventions shared by every entry point
 *   - Pointer ARRAYS (srcs, dsts, codes, scales) live in host memory and are
 *     read only during the call (copied by value into kernel arguments); the
 *     caller may free them on return. Every pointer IN them is a device
 *     pointer.
 *   - The caller owns all device memory. The library allocates nothing and
 *     keeps no state beyond a per-device cache of the compute-unit count,
 *     and (rx_allreduce_local_noalloc only) one static scratch array per
 *     device with its address.
 *   - Calls are stream-ordered and asynchronous: they return after enqueueing
 *     on `stream` (0 = the null stream). Synchronize the stream to observe
 *     results.
 *   - Validation happens before any HIP call; on any error nothing is
 *     enqueued. count == 0 returns RX_OK without launching anything.
 *   - Data buffers (sources, destinations, FP8 code buffers, high-precision
 *     outputs) must be 16-byte aligned; scale arrays 4-byte aligned.
 *   - Exact aliasing of an output with a source of the same element is
 *     allowed where stated (each element is read from every source before
 *     the same thread writes it); any partial overlap is undefined.
 *   - Sums are FP32, folded left in source order 0..nsrc-1 starting from
 *     source 0, one FP32 rounding per addition; BF16 results are rounded to
 *     nearest even. No NaN/Inf inputs are supported.
 *   - Stateless and reentrant; concurrent calls on different streams are
 *     independent.
 *   - Environment: RX_DEBUG=1 (read once per process) prints every launch's
 *     kernel, grid and workgroup size, and the HIP error of a failed
 *     launch, to stderr. RX_LOW_PRECISION_ENABLE=1 lets rx_allreduce_local's
 *     RX_ALGO_AUTO choose the low-precision algorithm. Nothing else is read.
 */
#ifndef RX_H
#define RX_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RX_FP32 = 0,     /* IEEE binary32                                        */
    RX_BF16 = 1,     /* bfloat16                                             */
    RX_FP8_E4M3 = 2, /* OCP E4M3 (E4M3FN): bias 7, max 448, no Inf           */
    RX_FP8_E5M2 = 3  /* OCP E5M2: bias 15, max 57344                         */
} rx_dtype_t;

typedef enum {
    RX_OK = 0,
    RX_ERR_NULL = 1,  /* a required pointer or pointer array is NULL        */
    RX_ERR_ARG = 2,   /* nsrc, rank, block or mode/pointer combination      */
    RX_ERR_DTYPE = 3, /* dtype not supported by this operation              */
    RX_ERR_ALIGN = 4, /* data buffer not 16-B aligned / scales not 4-B      */
    RX_ERR_HIP = 5,   /* the HIP runtime reported an error at launch        */
    RX_ERR_SCRATCH = 6 /* rx_allreduce_local_noalloc: the call needs more
                          than RX_NOALLOC_SCRATCH_BYTES of scratch          */
} rx_status_t;

typedef enum {
    RX_DRR_SUM = 0,     /* dequantize + FP32 sum -> high-precision output     */
    RX_DRR_REQUANT = 1  /* dequantize + FP32 sum -> requantized FP8 (+ hp)    */
} rx_drr_mode_t;

#define RX_MAX_SRC 16

/*
 * DDA flat, one rank's local reduce. Each rank reads every peer's buffer
 * directly and reduces locally, which turns an O(N)-step allreduce into one
 * step for small messages (RCCLX article, "Core feature 1: Direct Data
 * Access (DDA)", DDA Flat item); SUM with FP32 accumulation ("Core feature
 * 2: Low-Precision Collectives", feature table row "Compute precision";
 * "Practical guide", usage example).
 *
 *   dst[i] = cast( (((x_0[i] + x_1[i]) + x_2[i]) + ... ) + x_{nsrc-1}[i] )
 *
 * srcs   : nsrc device pointers, each `count` elements of `dtype`.
 * nsrc   : 1 .. RX_MAX_SRC.
 * dtype  : RX_FP32 or RX_BF16 (sources and dst share it).
 * dst    : `count` elements of `dtype`; may equal one srcs[j] exactly
 *          (in-place allreduce).
 */
rx_status_t rx_reduce_flat(const void* const* srcs, int nsrc, size_t count,
                           rx_dtype_t dtype, void* dst, hipStream_t stream);

/*
 * DDA tree, one rank's step: the reduce-scatter phase reduces this rank's
 * chunk across all sources, and the all-gather phase pushes the reduced
 * chunk into every destination, both by direct access (RCCLX article, "Core
 * feature 1: Direct Data Access (DDA)", DDA Tree item). Each rank reads and
 * writes one message's worth of bytes, the same volume as a ring.
 *
 * Chunking (the pages do not fix it): c = roundup(ceil(count/nsrc), V) with
 * V = 16 / sizeof(dtype), so every chunk starts 16-B aligned; chunk k is
 * [min(k c, count), min(k c + c, count)) and trailing ranks may own a short
 * or empty chunk. rx_tree_chunk() returns the bounds.
 *
 * srcs   : nsrc device pointers, each `count` elements of `dtype`.
 * rank   : 0 .. nsrc-1, the chunk this call reduces.
 * dsts   : nsrc device pointers, each `count` elements of `dtype`; only the
 *          chunk is written, everything outside it is left untouched.
 *          dsts[j] may equal srcs[j] exactly.
 */
rx_status_t rx_reduce_scatter_chunk_bcast(const void* const* srcs, int nsrc,
                                          size_t count, rx_dtype_t dtype,
                                          int rank, void* const* dsts,
                                          hipStream_t stream);

/* Host helper: bounds [*lo, *hi) of chunk `rank` (no HIP call). */
rx_status_t rx_tree_chunk(size_t count, int nsrc, rx_dtype_t dtype, int rank,
                          size_t* lo, size_t* hi);

/*
 * Low-precision path, sender side: FP32/BF16 -> FP8 with one FP32 scale per
 * block, up to 4:1 compression (RCCLX article, "Core feature 2:
 * Low-Precision Collectives", opening paragraph and feature table row "Data
 * types"). The pages do not give the encoding; this library fixes:
 *   block b = elements [b*block, min((b+1)*block, count)) of each source,
 *   A = max |x| over the block,
 *   s = A / FMAX, r = FMAX / A (each the correctly rounded FP32 quotient),
 *   (A == 0, s == 0 or r not finite: s = r = 1),
 *   code_i = OCP FP8 of fl32(x_i * r), round to nearest even, saturating.
 *
 * srcs      : nsrc device pointers, `count` elements of src_dtype each.
 * src_dtype : RX_FP32 or RX_BF16.
 * fp8_dtype : RX_FP8_E4M3 or RX_FP8_E5M2.
 * block     : 32, 64, 128, 256, 512 or 1024.
 * codes     : nsrc device pointers, `count` bytes each (16-B aligned).
 * scales    : nsrc device pointers, ceil(count/block) floats each.
 * Codes and scales must not overlap the sources.
 * RX_ERR_ARG also when (count / 256 + 1) * nsrc >= 2^32 (far beyond the
 * device memory of one GPU).
 */
rx_status_t rx_quant_fp8(const void* const* srcs, int nsrc, size_t count,
                         rx_dtype_t src_dtype, rx_dtype_t fp8_dtype, int block,
                         void* const* codes, float* const* scales,
                         hipStream_t stream);

/*
 * Low-precision path, reducing side: dequantize nsrc FP8 inputs, sum them in
 * FP32 (RCCLX article, "Core feature 2: Low-Precision Collectives", table row
 * "Compute precision"), and either return the sum or requantize it for the
 * all-gather.
 *   v_{r,i} = fl32(decode(code_{r,i}) * s_{r,b})      (never fused with +)
 *   S_i     = left fold of v_{0,i} .. v_{nsrc-1,i} in FP32
 *   RX_DRR_SUM     : out_hp[i] = cast(S_i). out_hp required; out_codes and
 *                    out_scales must be NULL.
 *   RX_DRR_REQUANT : S is quantized per block exactly as rx_quant_fp8 does
 *                    (same block and fp8_dtype) into out_codes/out_scales
 *                    (both required). When out_hp is not NULL it receives
 *                    cast(fl32(decode(out_code_i) * out_scale_b)), the value
 *                    every rank holds after the all-gather.
 * With nsrc == 1 and RX_DRR_SUM this is a plain dequantization.
 *
 * codes, scales : nsrc device pointers each (`count` bytes, ceil(count/block)
 *                 floats).
 * fp8_dtype     : RX_FP8_E4M3 or RX_FP8_E5M2; block as for rx_quant_fp8.
 * hp_dtype      : RX_FP32 or RX_BF16 (checked only when out_hp != NULL).
 * Outputs must not overlap the inputs.
 */
rx_status_t rx_dequant_reduce_requant(const void* const* codes,
                                      const float* const* scales, int nsrc,
                                      size_t count, rx_dtype_t fp8_dtype,
                                      int block, rx_drr_mode_t mode,
                                      void* out_codes, float* out_scales,
                                      void* out_hp, rx_dtype_t hp_dtype,
                                      hipStream_t stream);

/*
 * Low-precision tree step: one rank's share of a low-precision
 * reduce-scatter + all-gather, i.e. the DDA tree split (RCCLX article, "Core
 * feature 1: Direct Data Access (DDA)", DDA Tree item) applied to the FP8
 * messages of the low-precision collectives ("Core feature 2: Low-Precision
 * Collectives", which lists ReduceScatter and AllGather among the supported
 * operations). This rank dequantizes its chunk of every rank's codes, sums in
 * FP32, requantizes exactly as rx_dequant_reduce_requant does, and pushes the
 * FP8 codes and scales of the chunk into every destination.
 *
 * Chunks are whole scale blocks (the pages do not fix the split):
 * c = roundup(ceil(count/nsrc), block); chunk k = [min(k c, count),
 * min(k c + c, count)); rx_lp_tree_chunk() returns the bounds.
 *
 * codes, scales         : nsrc device pointers (count bytes, ceil(count/block)
 *                         floats), the ranks' quantized messages.
 * rank                  : 0 .. nsrc-1, the chunk this call reduces.
 * dst_codes, dst_scales : nsrc device pointers each, message-indexed like the
 *                         inputs; only chunk `rank` (codes) and its blocks
 *                         (scales) are written.
 * out_hp                : optional (NULL): chunk `rank` of the dequantized
 *                         result, hp_dtype RX_FP32 or RX_BF16, message-indexed.
 * Exact aliasing dst_codes[j] == codes[j] with dst_scales[j] == scales[j] is
 * allowed (in-place all-gather: every block is read completely by one wave
 * before that wave writes it); any other overlap is undefined.
 */
rx_status_t rx_lp_reduce_scatter_chunk_bcast(const void* const* codes,
                                             const float* const* scales, int nsrc,
                                             size_t count, rx_dtype_t fp8_dtype,
                                             int block, int rank,
                                             void* const* dst_codes,
                                             float* const* dst_scales,
                                             void* out_hp, rx_dtype_t hp_dtype,
                                             hipStream_t stream);

/* Host helper: bounds [*lo, *hi) of low-precision chunk `rank` (no HIP call). */
rx_status_t rx_lp_tree_chunk(size_t count, int nsrc, int block, int rank,
                             size_t* lo, size_t* hi);

typedef enum {
    RX_ALGO_AUTO = 0,    /* LOWPREC when enabled and >= 16 MiB, else FLAT   */
    RX_ALGO_FLAT = 1,    /* one fused sum-and-broadcast pass                */
    RX_ALGO_TREE = 2,    /* nsrc tree steps, one per rank's chunk           */
    RX_ALGO_LOWPREC = 3  /* quantize, nsrc low-precision tree steps, dequant */
} rx_algo_t;

/*
 * Allreduce (SUM) of nsrc rank buffers held on this device, in place:
 * afterwards every bufs[j] holds the result (RCCLX article, "Practical
 * guide": allreduce with ReduceOp.SUM, in place). It runs one of the
 * algorithms of the article on the local buffers:
 *   RX_ALGO_FLAT    each rank's result is the full reduce ("Core feature 1",
 *                   DDA Flat); on one device the nsrc identical reductions
 *                   are one pass that reads every buffer once and writes the
 *                   FP32 left fold into all of them.
 *   RX_ALGO_TREE    rx_reduce_scatter_chunk_bcast for every rank k in turn
 *                   ("Core feature 1", DDA Tree); same result as FLAT.
 *   RX_ALGO_LOWPREC every rank's rx_quant_fp8, then what every rank's
 *                   rx_lp_reduce_scatter_chunk_bcast and its dequantization
 *                   of the gathered FP8 message compute ("Core feature 2"):
 *                   every buffer receives dequant(requant(FP32 sum of the
 *                   dequantized inputs)). All of it is block-local, so on one
 *                   device it runs as one pass that keeps the codes in
 *                   registers when a block spans at most 64 16-byte vectors
 *                   (FP32 blocks up to 256, BF16 up to 512); larger blocks
 *                   quantize into the workspace first, then run one pass.
 *   RX_ALGO_AUTO    RX_ALGO_LOWPREC when the environment variable
 *                   RX_LOW_PRECISION_ENABLE is "1" and a buffer is >= 16 MiB
 *                   (the article's activation switch and threshold),
 *                   otherwise RX_ALGO_FLAT (on one device the flat pass is
 *                   never slower than nsrc tree steps).
 *
 * bufs            : nsrc device pointers, `count` elements of dtype each
 *                   (RX_FP32 or RX_BF16), 16-B aligned, distinct.
 * fp8_dtype, block: low-precision format and block size (as rx_quant_fp8);
 *                   checked only when the low-precision algorithm runs.
 * workspace       : device memory of at least rx_allreduce_local_workspace()
 *                   bytes, 256-B aligned; required by the low-precision
 *                   algorithm (NULL otherwise), written only for blocks
 *                   beyond the one-pass limit; its contents on return are
 *                   unspecified.
 * Errors: RX_ERR_NULL when the low-precision algorithm runs without a
 * workspace, RX_ERR_ARG when it is too small, as well as the errors of the
 * entry points above.
 */
rx_status_t rx_allreduce_local(void* const* bufs, int nsrc, size_t count,
                               rx_dtype_t dtype, rx_algo_t algo,
                               rx_dtype_t fp8_dtype, int block, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * rx_allreduce_local for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments, algorithms and results as rx_allreduce_local,
 * without the workspace: where the low-precision algorithm needs one (blocks
 * beyond its one-pass limit: FP32 blocks of 512 or 1024, BF16 blocks of
 * 1024), it keeps every rank's FP8 codes and scales in a scratch array
 * inside the library instead.
 *
 *   - The scratch holds RX_NOALLOC_SCRATCH_BYTES per device, allocated when
 *     the library's device code is loaded on that device and held until the
 *     process ends. A two-pass low-precision call whose
 *     rx_allreduce_local_workspace(nsrc, count, block) exceeds it returns
 *     RX_ERR_SCRATCH and enqueues nothing (e.g. 8 ranks of up to 8,355,840
 *     elements fit with blocks of 1024: 31 MiB of FP32 per rank). FLAT,
 *     TREE and the one-pass low-precision form use no scratch and have no
 *     such limit.
 *   - This entry point calls no hipMalloc, hipFree or other allocating
 *     routine. On its first call on a device (any algorithm, also with
 *     count == 0) it looks up that device's scratch address once
 *     (hipGetSymbolAddress, RX_ERR_HIP if that fails); make that first call
 *     outside a stream capture. Every later call uses the kept address.
 *   - Nothing in the scratch has to start at zero: the quantizer writes
 *     every code and scale the second pass reads. Its contents after a call
 *     are unspecified.
 *   - Every call on one device shares that device's scratch: calls that
 *     overlap in time on one device (different streams or host threads
 *     without ordering between them) race on it and give undefined results.
 *     Calls ordered on one stream are safe.
 */
#define RX_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
rx_status_t rx_allreduce_local_noalloc(void* const* bufs, int nsrc, size_t count,
                                       rx_dtype_t dtype, rx_algo_t algo,
                                       rx_dtype_t fp8_dtype, int block,
                                       hipStream_t stream);

/* Workspace bytes rx_allreduce_local needs for the low-precision algorithm
 * (codes and scales of every rank, each array 256-B aligned); 0 on invalid
 * arguments. No HIP call. */
size_t rx_allreduce_local_workspace(int nsrc, size_t count, int block);

/* Static description of a status code (never NULL). */
const char* rx_status_string(rx_status_t s);

#ifdef __cplusplus
}
#endif
#endif /* RX_H */
