/*
 * rx_oracle.c -- plain CPU oracle for the rx reduction library.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and
 * the benchmark's CPU-baseline leg, never by the product path. It shares no
 * code with the HIP library. Build: gcc -O2 -ffp-contract=off, no fast-math,
 * so every float expression below is one IEEE binary32 operation with
 * round-to-nearest-even.
 *
 * Sources of each definition are given per function; the readings taken
 * where the pages are silent are listed in rx_oracle.h.
 *
 * Pins: every function is pinned by tests that do not re-type its formula
 * (closed forms, brute-force nearest-value search, a library codec, the
 * pages' worked example, composition identities); nothing here is
 * "parity unpinned" except the NaN code chosen for NaN input, which the
 * pages and the library contract leave open.
 */
#include "rx_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------------- */
/* BF16 <-> FP32                                                           */
/* ---------------------------------------------------------------------- */

/* BF16 is the top half of an FP32 bit pattern, so widening is exact. */
float rxo_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Narrow to BF16 by keeping the top 16 bits and rounding on the 16 bits
 * dropped: above half a BF16 ulp rounds away from zero, below rounds toward
 * zero, exactly half rounds to the even BF16 pattern. NaN stays a (quiet)
 * NaN. A carry out of the mantissa bumps the exponent, which is also what
 * rounding to +-Inf needs. */
uint16_t rxo_f32_to_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if (isnan(x))
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t hi = u >> 16;
    uint32_t dropped = u & 0xFFFFu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (hi & 1u)))
        hi += 1u;
    return (uint16_t)hi;
}

/* ---------------------------------------------------------------------- */
/* OCP FP8 (E4M3 = E4M3FN, E5M2)                                           */
/* ---------------------------------------------------------------------- */

struct fp8_fmt {
    int ebits, mbits, bias;
    double fmax;
    uint8_t max_code; /* positive code of the largest finite value */
};

static struct fp8_fmt fmt_of(int fmt)
{
    struct fp8_fmt f;
    if (fmt == RXO_E4M3) {
        /* 4 exponent bits, bias 7, 3 mantissa bits; no infinities; only
         * S.1111.111 is NaN, so the largest finite is 1.75 * 2^8 = 448. */
        f.ebits = 4; f.mbits = 3; f.bias = 7; f.fmax = 448.0; f.max_code = 0x7E;
    } else {
        /* 5 exponent bits, bias 15, 2 mantissa bits; IEEE-like: exponent
         * field 31 is Inf/NaN, so the largest finite is 1.75 * 2^15. */
        f.ebits = 5; f.mbits = 2; f.bias = 15; f.fmax = 57344.0; f.max_code = 0x7B;
    }
    return f;
}

float rxo_fp8_max(int fmt) { return (float)fmt_of(fmt).fmax; }

/* Value of a code: sign, biased exponent, mantissa; exponent field 0 is the
 * subnormal range 0.m * 2^(1-bias). */
float rxo_fp8_decode(uint8_t code, int fmt)
{
    struct fp8_fmt f = fmt_of(fmt);
    int sign = code >> 7;
    int efield = (code >> f.mbits) & ((1 << f.ebits) - 1);
    int mfield = code & ((1 << f.mbits) - 1);
    double v;
    if (fmt == RXO_E4M3 && efield == 15 && mfield == 7)
        return NAN;
    if (fmt == RXO_E5M2 && efield == 31)
        return mfield == 0 ? (sign ? -INFINITY : INFINITY) : NAN;
    if (efield == 0)
        v = ldexp((double)mfield, 1 - f.bias - f.mbits);
    else
        v = ldexp((double)((1 << f.mbits) | mfield), efield - f.bias - f.mbits);
    return (float)(sign ? -v : v); /* exact: at most 4 significant bits */
}

/* Encode v: pick the binade of |v| (never below the smallest normal
 * exponent, which makes the subnormal range share its spacing), divide by
 * that binade's spacing, round the quotient to the nearest integer with ties
 * to even (rint in the default rounding mode), and assemble the code. Every
 * step in double is exact because v has 24 significant bits and the spacing
 * is a power of two. |v| >= FMAX (and +-Inf) saturate to +-FMAX. */
uint8_t rxo_fp8_encode(float v, int fmt)
{
    struct fp8_fmt f = fmt_of(fmt);
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v))
        return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    if (a >= f.fmax)
        return (uint8_t)(sign | f.max_code);

    int emin = 1 - f.bias; /* exponent of the smallest normal */
    int e = emin;
    if (a > 0.0) {
        int fe;
        frexp(a, &fe); /* a = m * 2^fe, m in [0.5, 1) */
        if (fe - 1 > emin)
            e = fe - 1;
    }
    double spacing = ldexp(1.0, e - f.mbits);
    double n = rint(a / spacing); /* integer in [0, 2^(mbits+1)] */
    int efield, mfield;
    if (n >= (double)(1 << (f.mbits + 1))) { /* carried into the next binade */
        e += 1;
        n = (double)(1 << f.mbits);
    }
    if (n < (double)(1 << f.mbits)) { /* subnormal (only when e == emin) */
        efield = 0;
        mfield = (int)n;
    } else {
        efield = e + f.bias;
        mfield = (int)n - (1 << f.mbits);
    }
    return (uint8_t)(sign | (efield << f.mbits) | mfield);
}

void rxo_fp8_encode_array(const float* in, size_t n, int fmt, uint8_t* out)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = rxo_fp8_encode(in[i], fmt);
}

void rxo_fp8_encode_bits_range(uint32_t first, uint32_t n, int fmt, uint8_t* out)
{
    for (uint32_t i = 0; i < n; ++i) {
        uint32_t u = first + i;
        float x;
        memcpy(&x, &u, sizeof x);
        out[i] = rxo_fp8_encode(x, fmt);
    }
}

void rxo_f32_to_bf16_array(const float* in, size_t n, uint16_t* out)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = rxo_f32_to_bf16(in[i]);
}

void rxo_fp8_decode_array(const uint8_t* in, size_t n, int fmt, float* out)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = rxo_fp8_decode(in[i], fmt);
}

/* ---------------------------------------------------------------------- */
/* Element access                                                          */
/* ---------------------------------------------------------------------- */

static float load_elem(const void* p, int dtype, size_t i)
{
    if (dtype == RXO_BF16)
        return rxo_bf16_to_f32(((const uint16_t*)p)[i]);
    return ((const float*)p)[i];
}

static void store_elem(void* p, int dtype, size_t i, float v)
{
    if (dtype == RXO_BF16)
        ((uint16_t*)p)[i] = rxo_f32_to_bf16(v);
    else
        ((float*)p)[i] = v;
}

static size_t elem_size(int dtype) { return dtype == RXO_BF16 ? 2u : 4u; }

/* ---------------------------------------------------------------------- */
/* DDA flat: local N-source reduce                                         */
/* ---------------------------------------------------------------------- */

/* One output element: widen every source to FP32 and fold left in source
 * order, one FP32 rounding per addition. */
static float fold_sources(const void* const* srcs, int nsrc, int dtype, size_t i)
{
    float acc = load_elem(srcs[0], dtype, i);
    for (int r = 1; r < nsrc; ++r) {
        float x = load_elem(srcs[r], dtype, i);
        acc = acc + x;
    }
    return acc;
}

/* Each rank reads every peer's buffer directly and reduces locally
 * (code-journey.com RCCLX article, "Core feature 1: DDA", DDA Flat item);
 * FP32 accumulation ("Core feature 2", table row "Compute precision"). */
void rxo_reduce_flat(const void* const* srcs, int nsrc, size_t count,
                     int dtype, void* dst)
{
    for (size_t i = 0; i < count; ++i)
        store_elem(dst, dtype, i, fold_sources(srcs, nsrc, dtype, i));
}

/* ---------------------------------------------------------------------- */
/* DDA tree: one rank's reduce-scatter chunk + all-gather push             */
/* ---------------------------------------------------------------------- */

void rxo_tree_chunk(size_t count, int nsrc, int dtype, int rank,
                    size_t* lo, size_t* hi)
{
    size_t per_vec = 16u / elem_size(dtype);
    size_t c = (count + (size_t)nsrc - 1) / (size_t)nsrc;
    c = (c + per_vec - 1) / per_vec * per_vec;
    size_t a = (size_t)rank * c;
    if (a > count) a = count;
    size_t b = a + c;
    if (b > count) b = count;
    *lo = a;
    *hi = b;
}

/* Reduce-scatter then all-gather, each by direct access (code-journey.com
 * RCCLX article, "Core feature 1: DDA", DDA Tree item): this rank reduces
 * only its chunk and pushes the result into every destination. */
void rxo_reduce_scatter_chunk_bcast(const void* const* srcs, int nsrc,
                                    size_t count, int dtype, int rank,
                                    void* const* dsts)
{
    size_t lo, hi;
    rxo_tree_chunk(count, nsrc, dtype, rank, &lo, &hi);
    for (size_t i = lo; i < hi; ++i) {
        float z = fold_sources(srcs, nsrc, dtype, i);
        for (int j = 0; j < nsrc; ++j)
            store_elem(dsts[j], dtype, i, z);
    }
}

/* ---------------------------------------------------------------------- */
/* Low-precision path                                                      */
/* ---------------------------------------------------------------------- */

void rxo_block_scale(const float* x, size_t len, int fmt, float* s, float* r)
{
    float fmax = rxo_fp8_max(fmt);
    float a = 0.0f;
    for (size_t i = 0; i < len; ++i) {
        float m = fabsf(x[i]);
        if (m > a) a = m;
    }
    if (a == 0.0f) {
        *s = 1.0f; *r = 1.0f;
        return;
    }
    float sv = a / fmax;
    float rv = fmax / a;
    if (sv == 0.0f || !isfinite(rv)) {
        *s = 1.0f; *r = 1.0f;
        return;
    }
    *s = sv;
    *r = rv;
}

void rxo_block_scale_bits_range(uint32_t first, uint32_t n, int fmt, float* s, float* r)
{
    for (uint32_t i = 0; i < n; ++i) {
        uint32_t u = first + i;
        float a;
        memcpy(&a, &u, sizeof a);
        rxo_block_scale(&a, 1, fmt, s + i, r + i);
    }
}

/* Quantize one block of FP32 values into codes and return its scale. */
static float quant_block(const float* x, size_t len, int fmt, uint8_t* codes)
{
    float s, r;
    rxo_block_scale(x, len, fmt, &s, &r);
    for (size_t i = 0; i < len; ++i) {
        float y = x[i] * r;
        codes[i] = rxo_fp8_encode(y, fmt);
    }
    return s;
}

/* FP32/BF16 -> FP8 with per-block scales (code-journey.com RCCLX article,
 * "Core feature 2: Low-Precision Collectives", opening paragraph and table
 * row "Data types"). */
void rxo_quant_fp8(const void* const* srcs, int nsrc, size_t count,
                   int src_dtype, int fmt, int block,
                   uint8_t* const* codes, float* const* scales)
{
    float* buf = (float*)malloc((size_t)block * sizeof(float));
    size_t nb = (count + (size_t)block - 1) / (size_t)block;
    for (int j = 0; j < nsrc; ++j) {
        for (size_t b = 0; b < nb; ++b) {
            size_t lo = b * (size_t)block;
            size_t len = count - lo < (size_t)block ? count - lo : (size_t)block;
            for (size_t i = 0; i < len; ++i)
                buf[i] = load_elem(srcs[j], src_dtype, lo + i);
            scales[j][b] = quant_block(buf, len, fmt, codes[j] + lo);
        }
    }
    free(buf);
}

/* Dequantize every source and fold in FP32 (table row "Compute precision"),
 * then either emit the sum or requantize it with the same block size and
 * format. */
void rxo_dequant_reduce_requant(const uint8_t* const* codes,
                                const float* const* scales, int nsrc,
                                size_t count, int fmt, int block, int mode,
                                uint8_t* out_codes, float* out_scales,
                                void* out_hp, int hp_dtype)
{
    float* sum = (float*)malloc((size_t)block * sizeof(float));
    uint8_t* cq = (uint8_t*)malloc((size_t)block);
    size_t nb = (count + (size_t)block - 1) / (size_t)block;
    for (size_t b = 0; b < nb; ++b) {
        size_t lo = b * (size_t)block;
        size_t len = count - lo < (size_t)block ? count - lo : (size_t)block;
        for (size_t i = 0; i < len; ++i) {
            float acc = rxo_fp8_decode(codes[0][lo + i], fmt) * scales[0][b];
            for (int r = 1; r < nsrc; ++r) {
                float v = rxo_fp8_decode(codes[r][lo + i], fmt) * scales[r][b];
                acc = acc + v;
            }
            sum[i] = acc;
        }
        if (mode == RXO_DRR_SUM) {
            for (size_t i = 0; i < len; ++i)
                store_elem(out_hp, hp_dtype, lo + i, sum[i]);
            continue;
        }
        float s2 = quant_block(sum, len, fmt, cq);
        out_scales[b] = s2;
        memcpy(out_codes + lo, cq, len);
        if (out_hp) {
            for (size_t i = 0; i < len; ++i) {
                float d = rxo_fp8_decode(cq[i], fmt) * s2;
                store_elem(out_hp, hp_dtype, lo + i, d);
            }
        }
    }
    free(cq);
    free(sum);
}

/* ---------------------------------------------------------------------- */
/* Low-precision tree step                                                 */
/* ---------------------------------------------------------------------- */

void rxo_lp_tree_chunk(size_t count, int nsrc, int block, int rank,
                       size_t* lo, size_t* hi)
{
    size_t c = (count + (size_t)nsrc - 1) / (size_t)nsrc;
    c = (c + (size_t)block - 1) / (size_t)block * (size_t)block;
    size_t a = (size_t)rank * c;
    if (a > count) a = count;
    size_t b = a + c;
    if (b > count) b = count;
    *lo = a;
    *hi = b;
}

/* The reduce-scatter / all-gather split of the DDA tree item of the RCCLX
 * article ("Core feature 1") carried out on the FP8 messages of "Core
 * feature 2": this rank reduces its chunk of every rank's codes in FP32,
 * requantizes it, and pushes the FP8 chunk to every rank. */
void rxo_lp_reduce_scatter_chunk_bcast(const uint8_t* const* codes,
                                       const float* const* scales, int nsrc,
                                       size_t count, int fmt, int block,
                                       int rank, uint8_t* const* dst_codes,
                                       float* const* dst_scales,
                                       void* out_hp, int hp_dtype)
{
    size_t lo, hi;
    rxo_lp_tree_chunk(count, nsrc, block, rank, &lo, &hi);
    if (lo >= hi || nsrc > 64)
        return;
    size_t len = hi - lo;
    size_t nb = (len + (size_t)block - 1) / (size_t)block;
    size_t b0 = lo / (size_t)block;
    const uint8_t* csub[64];
    const float* ssub[64];
    for (int r = 0; r < nsrc; ++r) {
        csub[r] = codes[r] + lo;
        ssub[r] = scales[r] + b0;
    }
    uint8_t* oc = (uint8_t*)malloc(len);
    float* os = (float*)malloc(nb * sizeof(float));
    void* hp = NULL;
    if (out_hp)
        hp = (uint8_t*)out_hp + lo * elem_size(hp_dtype);
    rxo_dequant_reduce_requant(csub, ssub, nsrc, len, fmt, block, RXO_DRR_REQUANT,
                               oc, os, hp, hp_dtype);
    for (int j = 0; j < nsrc; ++j) {
        memcpy(dst_codes[j] + lo, oc, len);
        memcpy(dst_scales[j] + b0, os, nb * sizeof(float));
    }
    free(os);
    free(oc);
}

/* ---------------------------------------------------------------------- */
/* Local allreduce (all ranks' buffers on one device)                      */
/* ---------------------------------------------------------------------- */

/* The usage example of the RCCLX article ("Practical guide": allreduce with
 * ReduceOp.SUM, in place) carried out with each of the algorithms of "Core
 * feature 1" (DDA flat, DDA tree) and "Core feature 2" (low precision). */
void rxo_allreduce_local(void* const* bufs, int nsrc, size_t count, int dtype,
                         int algo, int fmt, int block)
{
    if (count == 0 || nsrc < 1 || nsrc > 64)
        return;
    size_t es = elem_size(dtype);
    if (algo == RXO_ALGO_FLAT || algo == RXO_ALGO_TREE) {
        void* y = malloc(count * es);
        rxo_reduce_flat((const void* const*)bufs, nsrc, count, dtype, y);
        for (int j = 0; j < nsrc; ++j)
            memcpy(bufs[j], y, count * es);
        free(y);
        return;
    }
    /* low precision */
    size_t nb = (count + (size_t)block - 1) / (size_t)block;
    uint8_t* codes[64];
    float* scales[64];
    for (int j = 0; j < nsrc; ++j) {
        codes[j] = (uint8_t*)malloc(count);
        scales[j] = (float*)malloc(nb * sizeof(float));
    }
    rxo_quant_fp8((const void* const*)bufs, nsrc, count, dtype, fmt, block, codes, scales);
    uint8_t* rc[64];
    float* rs[64];
    for (int j = 0; j < nsrc; ++j) {
        rc[j] = (uint8_t*)malloc(count);
        rs[j] = (float*)malloc(nb * sizeof(float));
    }
    for (int k = 0; k < nsrc; ++k)
        rxo_lp_reduce_scatter_chunk_bcast((const uint8_t* const*)codes, (const float* const*)scales,
                                          nsrc, count, fmt, block, k, rc, rs, NULL, RXO_FP32);
    for (int j = 0; j < nsrc; ++j) {
        const uint8_t* cj[1] = {rc[j]};
        const float* sj[1] = {rs[j]};
        rxo_dequant_reduce_requant(cj, sj, 1, count, fmt, block, RXO_DRR_SUM, NULL, NULL,
                                   bufs[j], dtype);
    }
    for (int j = 0; j < nsrc; ++j) {
        free(codes[j]); free(scales[j]); free(rc[j]); free(rs[j]);
    }
}
