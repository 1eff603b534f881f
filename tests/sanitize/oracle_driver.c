/* Runs every CPU-oracle entry point over ragged shapes with buffers of
 * exactly the documented sizes, so that a host build with address and
 * undefined-behaviour checking reports any out-of-bounds access, leak or
 * undefined operation. Prints "ok" and exits 0 when every call returned and
 * the rank-id example summed to N(N-1)/2. Test infrastructure only. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/rx_oracle.h"

static void* xmalloc(size_t n)
{
    void* p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static size_t esz(int dtype) { return dtype == RXO_BF16 ? 2 : 4; }

/* deterministic values in [-4, 4), stored as FP32 or BF16 */
static void fill(void* p, size_t count, int dtype, unsigned seed)
{
    unsigned s = seed * 2654435761u + 12345u;
    for (size_t i = 0; i < count; ++i) {
        s = s * 1664525u + 1013904223u;
        float v = (float)((s >> 8) & 0xFFFF) / 8192.0f - 4.0f;
        if (dtype == RXO_BF16)
            ((uint16_t*)p)[i] = rxo_f32_to_bf16(v);
        else
            ((float*)p)[i] = v;
    }
}

static int run_shape(int n, size_t count, int dtype, int fmt, int block)
{
    const size_t nb = (count + (size_t)block - 1) / (size_t)block;
    void* src[16];
    void* dst[16];
    uint8_t* codes[16];
    float* scales[16];
    uint8_t* dcodes[16];
    float* dscales[16];
    for (int j = 0; j < n; ++j) {
        src[j] = xmalloc(count * esz(dtype));
        dst[j] = xmalloc(count * esz(dtype));
        codes[j] = (uint8_t*)xmalloc(count);
        scales[j] = (float*)xmalloc(nb * sizeof(float));
        dcodes[j] = (uint8_t*)xmalloc(count);
        dscales[j] = (float*)xmalloc(nb * sizeof(float));
        fill(src[j], count, dtype, (unsigned)(j + 1));
        memset(dst[j], 0, count * esz(dtype));
        memset(dcodes[j], 0, count);
        memset(dscales[j], 0, nb * sizeof(float));
    }
    void* flat = xmalloc(count * esz(dtype));
    rxo_reduce_flat((const void* const*)src, n, count, dtype, flat);
    for (int k = 0; k < n; ++k) {
        size_t lo, hi;
        rxo_tree_chunk(count, n, dtype, k, &lo, &hi);
        rxo_reduce_scatter_chunk_bcast((const void* const*)src, n, count, dtype, k, dst);
    }
    rxo_quant_fp8((const void* const*)src, n, count, dtype, fmt, block, codes, scales);
    uint8_t* oc = (uint8_t*)xmalloc(count);
    float* os = (float*)xmalloc(nb * sizeof(float));
    void* hp = xmalloc(count * esz(dtype));
    rxo_dequant_reduce_requant((const uint8_t* const*)codes, (const float* const*)scales, n, count,
                               fmt, block, RXO_DRR_REQUANT, oc, os, hp, dtype);
    rxo_dequant_reduce_requant((const uint8_t* const*)codes, (const float* const*)scales, n, count,
                               fmt, block, RXO_DRR_SUM, NULL, NULL, hp, dtype);
    rxo_dequant_reduce_requant((const uint8_t* const*)&oc, (const float* const*)&os, 1, count,
                               fmt, block, RXO_DRR_SUM, NULL, NULL, hp, dtype);
    for (int k = 0; k < n; ++k) {
        size_t lo, hi;
        rxo_lp_tree_chunk(count, n, block, k, &lo, &hi);
        rxo_lp_reduce_scatter_chunk_bcast((const uint8_t* const*)codes, (const float* const*)scales,
                                          n, count, fmt, block, k, dcodes, dscales,
                                          k == 0 ? hp : NULL, dtype);
    }
    for (int algo = RXO_ALGO_FLAT; algo <= RXO_ALGO_LOWPREC; ++algo)
        rxo_allreduce_local(dst, n, count, dtype, algo, fmt, block);
    free(flat);
    free(oc);
    free(os);
    free(hp);
    for (int j = 0; j < n; ++j) {
        free(src[j]);
        free(dst[j]);
        free(codes[j]);
        free(scales[j]);
        free(dcodes[j]);
        free(dscales[j]);
    }
    return 0;
}

int main(void)
{
    static const int ns[] = {1, 2, 3, 8, 13, 16};
    static const size_t counts[] = {1, 7, 8, 17, 255, 257, 1000, 4133};
    static const int blocks[] = {32, 128, 256, 1024};
    for (size_t a = 0; a < sizeof ns / sizeof ns[0]; ++a)
        for (size_t b = 0; b < sizeof counts / sizeof counts[0]; ++b)
            for (size_t c = 0; c < sizeof blocks / sizeof blocks[0]; ++c)
                for (int dtype = RXO_FP32; dtype <= RXO_BF16; ++dtype)
                    run_shape(ns[a], counts[b], dtype, (int)((a + b + c) % 2) ? RXO_E5M2 : RXO_E4M3,
                              blocks[c]);

    /* the rank-id example: 8 ranks of 10 x 20 FP32, SUM -> 28 everywhere */
    float* bufs[8];
    for (int r = 0; r < 8; ++r) {
        bufs[r] = (float*)xmalloc(200 * sizeof(float));
        for (int i = 0; i < 200; ++i) bufs[r][i] = (float)r;
    }
    float* y = (float*)xmalloc(200 * sizeof(float));
    rxo_reduce_flat((const void* const*)bufs, 8, 200, RXO_FP32, y);
    int bad = 0;
    for (int i = 0; i < 200; ++i) bad |= y[i] != 28.0f;
    free(y);
    for (int r = 0; r < 8; ++r) free(bufs[r]);
    if (bad) {
        fprintf(stderr, "rank-id example did not sum to 28\n");
        return 1;
    }
    printf("ok\n");
    return 0;
}
