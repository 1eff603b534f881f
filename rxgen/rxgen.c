/*
 * rxgen.c -- seeded synthetic inputs for the rx library's tests and bench.
 *
 * This module only draws input values; it holds none of the reduction,
 * quantization or rounding arithmetic that the library and the oracle
 * compute. Both sides read the bytes it writes.
 *
 * Generator: splitmix64 (Vigna's published 64-bit mixer) in counter mode.
 *   key(seed, rank, stream) = mix(seed * 2^32 + rank + stream * 2^24)
 *   h(i)                    = mix(key + i)
 * so element i depends only on (seed, rank, stream, i): the result does not
 * depend on how many threads fill the buffer, and any sub-range can be
 * generated on its own (the `offset` argument).
 *
 * Distributions (element i, 53-bit uniforms from h):
 *   RXG_RANK      x = rank
 *   RXG_UNIFORM   x = (h >> 40) * 2^-23 - 1            (24-bit grid on [-1,1))
 *   RXG_NORMAL    Box-Muller on the pair p = i / 2:
 *                 u1 = ((h(2p) >> 11) + 1) 2^-53, u2 = (h(2p+1) >> 11) 2^-53,
 *                 x = sqrt(-2 ln u1) * (cos | sin)(2 pi u2) for even | odd i
 *   RXG_NORMAL_OUTLIER   RXG_NORMAL, then x *= 100 when an independent
 *                 stream's h(i) < 0.01 * 2^64 (1% outliers, times 100)
 *   RXG_LAPLACE   u = ((h >> 11) + 0.5) 2^-53 - 0.5, x = -sgn(u) ln(1 - 2|u|)
 *   RXG_INT       x = integer uniform in [-param, param] (exact in FP32 for
 *                 param <= 2^24)
 * Values are computed in double and rounded once to FP32. BF16 output keeps
 * the top 16 bits of that FP32 pattern (truncation), a generator-side
 * choice that only shapes the input distribution.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>
#include <unistd.h>

enum { RXG_FP32 = 0, RXG_BF16 = 1 };
enum {
    RXG_RANK = 0,
    RXG_UNIFORM = 1,
    RXG_NORMAL = 2,
    RXG_NORMAL_OUTLIER = 3,
    RXG_LAPLACE = 4,
    RXG_INT = 5
};

uint64_t rxg_mix(uint64_t z)
{
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static uint64_t key_of(uint64_t seed, int rank, int stream)
{
    return rxg_mix((seed << 32) + (uint64_t)(uint32_t)rank + ((uint64_t)stream << 24));
}

static double u53_open0(uint64_t h) { return (double)((h >> 11) + 1) * 0x1p-53; }
static double u53(uint64_t h) { return (double)(h >> 11) * 0x1p-53; }

static double sample(int dist, uint64_t key, uint64_t key_o, int rank,
                     int64_t param, uint64_t i)
{
    static const double two_pi = 6.283185307179586476925286766559;
    switch (dist) {
    case RXG_RANK:
        return (double)rank;
    case RXG_UNIFORM:
        return (double)(rxg_mix(key + i) >> 40) * 0x1p-23 - 1.0;
    case RXG_NORMAL:
    case RXG_NORMAL_OUTLIER: {
        uint64_t p = i >> 1;
        double u1 = u53_open0(rxg_mix(key + 2 * p));
        double u2 = u53(rxg_mix(key + 2 * p + 1));
        double rad = sqrt(-2.0 * log(u1));
        double z = (i & 1) ? rad * sin(two_pi * u2) : rad * cos(two_pi * u2);
        if (dist == RXG_NORMAL_OUTLIER) {
            /* 0.01 * 2^64, rounded down */
            if (rxg_mix(key_o + i) < 184467440737095516ull)
                z *= 100.0;
        }
        return z;
    }
    case RXG_LAPLACE: {
        double u = ((double)(rxg_mix(key + i) >> 11) + 0.5) * 0x1p-53 - 0.5;
        double a = -log(1.0 - 2.0 * fabs(u));
        return u < 0 ? -a : a;
    }
    case RXG_INT: {
        uint64_t span = (uint64_t)(2 * param + 1);
        return (double)((int64_t)(rxg_mix(key + i) % span) - param);
    }
    default:
        return 0.0;
    }
}

struct job {
    void* dst;
    int dtype, dist, rank;
    uint64_t key, key_o;
    int64_t param;
    uint64_t offset;
    size_t lo, hi;
};

static void* run_job(void* arg)
{
    struct job* j = (struct job*)arg;
    for (size_t i = j->lo; i < j->hi; ++i) {
        float f = (float)sample(j->dist, j->key, j->key_o, j->rank, j->param,
                                j->offset + i);
        if (j->dtype == RXG_BF16) {
            uint32_t u;
            memcpy(&u, &f, sizeof u);
            ((uint16_t*)j->dst)[i] = (uint16_t)(u >> 16);
        } else {
            ((float*)j->dst)[i] = f;
        }
    }
    return NULL;
}

/* Fill dst[0 .. count) with samples offset .. offset + count of the stream
 * (seed, rank). nthreads <= 0 picks min(16, online CPUs). Returns 0, or -1
 * on a bad argument. */
int rxg_fill(void* dst, size_t count, int dtype, int dist, uint64_t seed,
             int rank, int64_t param, uint64_t offset, int nthreads)
{
    if (!dst && count)
        return -1;
    if (dtype != RXG_FP32 && dtype != RXG_BF16)
        return -1;
    if (dist < RXG_RANK || dist > RXG_INT)
        return -1;
    if (nthreads <= 0) {
        long c = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = c > 16 ? 16 : (c < 1 ? 1 : (int)c);
    }
    if ((size_t)nthreads > count / 65536 + 1)
        nthreads = (int)(count / 65536 + 1);
    if (nthreads > 64)
        nthreads = 64;

    struct job jobs[64];
    pthread_t tids[64];
    uint64_t key = key_of(seed, rank, 0);
    uint64_t key_o = key_of(seed, rank, 1);
    size_t per = (count + (size_t)nthreads - 1) / (size_t)nthreads;
    for (int t = 0; t < nthreads; ++t) {
        size_t lo = (size_t)t * per;
        size_t hi = lo + per;
        if (lo > count) lo = count;
        if (hi > count) hi = count;
        jobs[t] = (struct job){dst, dtype, dist, rank, key, key_o, param, offset, lo, hi};
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tids[t], NULL, run_job, &jobs[t]) != 0)
            break;
        started = t;
    }
    run_job(&jobs[0]);
    for (int t = started + 1; t < nthreads; ++t)
        run_job(&jobs[t]); /* threads that failed to start run inline */
    for (int t = 1; t <= started; ++t)
        pthread_join(tids[t], NULL);
    return 0;
}
