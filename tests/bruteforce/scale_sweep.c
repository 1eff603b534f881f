/*
 * scale_sweep.c -- exhaustive check of the oracle's block scale (test
 * infrastructure, host code only).
 *
 * For every non-negative finite FP32 block absmax A, the oracle returns
 * s = fl32(A / FMAX) and r = fl32(FMAX / A), or s = r = 1 for a degenerate
 * block (A == 0, s rounds to 0, or r overflows). This file checks both
 * against the definition of a correctly rounded division, with exact
 * arithmetic: q is the correctly rounded quotient N / D iff N lies between
 * D times the midpoints from q to its two FP32 neighbours, and on a
 * midpoint q has an even significand. A midpoint has at most 25 significant
 * bits and D at most 24, so each product is exact in double precision.
 * Degeneracy is decided the same way: s rounds to 0 iff A / FMAX <= 2^-150
 * (a tie rounds to the even 0), r overflows iff FMAX / A >= FLT_MAX plus
 * half its spacing. The oracle is called through the function pointer the
 * caller passes (its bits-range entry point), over disjoint ranges of A on
 * worker threads.
 */
#include <float.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

typedef void (*range_fn)(uint32_t first, uint32_t n, int fmt, float* s, float* r);

struct job {
    range_fn fn;
    int fmt;
    double fmax;
    uint32_t lo, hi; /* A bit patterns [lo, hi) */
    uint64_t checked, bad;
    uint32_t first_bad;
};

static float f_of(uint32_t u) { float f; memcpy(&f, &u, sizeof f); return f; }
static uint32_t bits_of(float f) { uint32_t u; memcpy(&u, &f, sizeof u); return u; }

/* q == correctly rounded n / d (n, d > 0 finite; q finite and > 0). */
static int rounded_ok(float q, double n, double d)
{
    if (!(q > 0.0f) || !isfinite(q))
        return 0;
    double qd = q;
    float below = nextafterf(q, 0.0f);
    float above = nextafterf(q, INFINITY);
    double lo_mid = (qd + (double)below) / 2.0;
    double hi_mid = isfinite(above) ? (qd + (double)above) / 2.0
                                    : qd + (qd - (double)below) / 2.0;
    double plo = lo_mid * d, phi = hi_mid * d; /* exact */
    int even = (bits_of(q) & 1u) == 0;
    if (n < plo || n > phi)
        return 0;
    if ((n == plo || n == phi) && !even)
        return 0;
    return 1;
}

static void* run(void* p)
{
    struct job* j = p;
    enum { CH = 1 << 16 };
    float s[CH], r[CH];
    const double fm = j->fmax;
    const double s_zero = ldexp(fm, -150);                   /* A <= this: s rounds to 0 */
    const double r_inf = ldexp(1.0, 128) - ldexp(1.0, 103);  /* FLT_MAX + half its spacing */
    for (uint64_t base = j->lo; base < j->hi; base += CH) {
        uint32_t n = (uint32_t)((j->hi - base) < CH ? (j->hi - base) : CH);
        j->fn((uint32_t)base, n, j->fmt, s, r);
        for (uint32_t k = 0; k < n; ++k) {
            const uint32_t bits = (uint32_t)base + k;
            const double a = (double)f_of(bits);
            const int degenerate = a == 0.0 || a <= s_zero || fm >= r_inf * a;
            int ok;
            if (degenerate)
                ok = s[k] == 1.0f && r[k] == 1.0f;
            else
                ok = rounded_ok(s[k], a, fm) && rounded_ok(r[k], fm, a);
            j->checked++;
            if (!ok) {
                if (j->bad == 0)
                    j->first_bad = bits;
                j->bad++;
            }
        }
    }
    return NULL;
}

/* Every A in [0, FLT_MAX]: returns 0, or -1 on a bad argument. */
int scale_sweep(int fmt, double fmax, void* range_entry, int nthreads, uint64_t* checked,
                uint64_t* bad, uint32_t* first_bad)
{
    if (nthreads < 1 || nthreads > 64 || !range_entry || !(fmax > 0.0))
        return -1;
    const uint64_t total = (uint64_t)bits_of(FLT_MAX) + 1;
    struct job jobs[64];
    pthread_t th[64];
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = (struct job){(range_fn)range_entry, fmt, fmax,
                               (uint32_t)(total * i / nthreads),
                               (uint32_t)(total * (i + 1) / nthreads), 0, 0, 0};
        pthread_create(&th[i], NULL, run, &jobs[i]);
    }
    *checked = 0;
    *bad = 0;
    *first_bad = 0;
    for (int i = 0; i < nthreads; ++i) {
        pthread_join(th[i], NULL);
        *checked += jobs[i].checked;
        if (jobs[i].bad && *bad == 0)
            *first_bad = jobs[i].first_bad;
        *bad += jobs[i].bad;
    }
    return 0;
}
