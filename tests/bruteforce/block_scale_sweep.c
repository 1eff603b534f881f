/*
 * block_scale_sweep.c -- host check of the arithmetic the kernels use for the
 * block scale (test infrastructure, host code only; not the oracle).
 *
 * The kernels form s = A / FMAX and r = FMAX / A without a division: FMA-
 * corrected products after P. Markstein ("IA-64 and Elementary Functions",
 * 2000), s from the constant RN(1 / FMAX), r from a hardware reciprocal
 * estimate of A / 4 refined by one Newton step, with FMAX / 4 over A / 4.
 * This file repeats those steps in host FP32 (fmaf, IEEE, no contraction)
 * and compares them, after the degenerate-block rule (A == 0, s == 0 or r
 * not finite -> s = r = 1), with the host's IEEE division, which is
 * correctly rounded. The hardware estimate is only known to lie within 1 ulp
 * of 1 / (A / 4), so every float within 1 ulp of the correctly rounded
 * reciprocal (it and both neighbours) is tried.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

static float bits_to_f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static void degenerate(float a, float sv, float rv, float* s, float* r)
{
    int d = (a == 0.0f) | (sv == 0.0f) | !isfinite(rv);
    *s = d ? 1.0f : sv;
    *r = d ? 1.0f : rv;
}

struct job {
    float fmax;
    uint32_t lo, hi, step;
    uint64_t checked, bad;
    uint32_t first;
};

static void* run(void* p)
{
    struct job* j = (struct job*)p;
    const float m = j->fmax;
    volatile float one = 1.0f;
    const float inv_m = one / m, m4 = 0.25f * m;
    for (uint64_t u = j->lo; u < j->hi; u += j->step) {
        const float a = bits_to_f((uint32_t)u);
        float S, R;
        degenerate(a, a / m, m / a, &S, &R);
        const float q0 = a * inv_m;
        float sv = fmaf(fmaf(-q0, m, a), inv_m, q0);
        const float a4 = 0.25f * a;
        const float yr = one / a4;
        const float ys[3] = {nextafterf(yr, 0.0f), yr, nextafterf(yr, INFINITY)};
        for (int k = 0; k < 3; ++k) {
            const float y1 = fmaf(fmaf(-a4, ys[k], 1.0f), ys[k], ys[k]);
            const float p0 = m4 * y1;
            float rv = fmaf(fmaf(-p0, a4, m4), y1, p0);
            const int inf = a == INFINITY;
            float s2, r2;
            degenerate(a, inf ? a : sv, inf ? 0.0f : rv, &s2, &r2);
            ++j->checked;
            if (f_to_bits(s2) != f_to_bits(S) || f_to_bits(r2) != f_to_bits(R)) {
                if (!j->bad || (uint32_t)u < j->first)
                    j->first = (uint32_t)u;
                ++j->bad;
            }
        }
    }
    return 0;
}

/* A bit patterns lo, lo + step, ... below hi, split over threads. Returns 0. */
int block_scale_sweep(float fmax, uint32_t lo, uint32_t hi, uint32_t step, int threads,
                      uint64_t* checked, uint64_t* bad, uint32_t* first)
{
    struct job jobs[64];
    pthread_t tid[64];
    if (threads < 1) threads = 1;
    if (threads > 64) threads = 64;
    const uint64_t n = ((uint64_t)hi - lo + step - 1) / step;
    const uint64_t per = (n + threads - 1) / threads;
    for (int t = 0; t < threads; ++t) {
        const uint64_t a = (uint64_t)lo + (uint64_t)t * per * step;
        const uint64_t b = a + per * step;
        jobs[t].fmax = fmax;
        jobs[t].lo = (uint32_t)(a < hi ? a : hi);
        jobs[t].hi = (uint32_t)(b < hi ? b : hi);
        jobs[t].step = step;
        jobs[t].checked = jobs[t].bad = 0;
        jobs[t].first = 0;
        pthread_create(&tid[t], 0, run, &jobs[t]);
    }
    *checked = *bad = 0;
    *first = 0;
    for (int t = 0; t < threads; ++t) {
        pthread_join(tid[t], 0);
        *checked += jobs[t].checked;
        if (jobs[t].bad && (!*bad || jobs[t].first < *first))
            *first = jobs[t].first;
        *bad += jobs[t].bad;
    }
    return 0;
}
