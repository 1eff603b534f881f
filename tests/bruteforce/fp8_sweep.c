/*
 * fp8_sweep.c -- exhaustive check of the oracle's FP8 encoder (test
 * infrastructure, host code only).
 *
 * Every FP32 bit pattern except the NaNs is encoded twice: by the encoder
 * passed in as a function pointer (the oracle's), and by an independent
 * nearest-value search over a decode table the caller supplies (torch's
 * float8 dtypes, not the oracle's decoder). The search takes the nearest
 * finite value, the even code on a tie, and clamps magnitudes at or beyond
 * the largest finite value to it (the saturating OCP conversion); the sign
 * bit is copied from the input, so -0 encodes as 0x80. The 2^32 patterns
 * are split into disjoint ranges over worker threads.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

typedef uint8_t (*enc_fn)(float, int);

struct table {
    double val[128];   /* finite non-negative values, ascending */
    uint8_t code[128]; /* their codes */
    int n;
};

struct job {
    const struct table* t;
    enc_fn enc;
    int fmt;
    uint64_t lo, hi;
    uint64_t checked, bad;
    uint32_t first_bad;
};

static uint8_t nearest(const struct table* t, float x)
{
    double a = fabs((double)x);
    if (a > t->val[t->n - 1])
        a = t->val[t->n - 1];
    int lo = 0, hi = t->n - 1; /* first index with val >= a */
    while (lo < hi) {
        int mid = (lo + hi) / 2;
        if (t->val[mid] >= a)
            hi = mid;
        else
            lo = mid + 1;
    }
    uint8_t c;
    if (t->val[hi] == a || hi == 0) {
        c = t->code[hi];
    } else {
        double d_lo = a - t->val[hi - 1], d_hi = t->val[hi] - a;
        int pick_hi = d_hi < d_lo || (d_hi == d_lo && (t->code[hi] & 1) == 0);
        c = pick_hi ? t->code[hi] : t->code[hi - 1];
    }
    return (uint8_t)(c | (signbit(x) ? 0x80 : 0x00));
}

static void* run(void* p)
{
    struct job* j = p;
    for (uint64_t u = j->lo; u < j->hi; ++u) {
        uint32_t bits = (uint32_t)u;
        float x;
        memcpy(&x, &bits, sizeof x);
        if (isnan(x))
            continue;
        uint8_t want = nearest(j->t, x);
        uint8_t got = j->enc(x, j->fmt);
        j->checked++;
        if (got != want) {
            if (j->bad == 0)
                j->first_bad = bits;
            j->bad++;
        }
    }
    return NULL;
}

/* decode256: value of every code (NaN for the NaN codes). Returns 0, or -1
 * on a bad argument. */
int fp8_sweep(const float* decode256, int fmt, void* encoder, int nthreads,
              uint64_t* checked, uint64_t* bad, uint32_t* first_bad)
{
    if (nthreads < 1 || nthreads > 64 || !decode256 || !encoder)
        return -1;
    struct table t;
    t.n = 0;
    for (int c = 0; c < 128; ++c) {
        if (!isfinite(decode256[c]))
            continue;
        /* insertion sort by value, codes ascending among equal values */
        int k = t.n++;
        while (k > 0 && t.val[k - 1] > (double)decode256[c]) {
            t.val[k] = t.val[k - 1];
            t.code[k] = t.code[k - 1];
            --k;
        }
        t.val[k] = (double)decode256[c];
        t.code[k] = (uint8_t)c;
    }
    struct job jobs[64];
    pthread_t th[64];
    const uint64_t total = (uint64_t)1 << 32;
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = (struct job){&t, (enc_fn)encoder, fmt, total * i / nthreads,
                               total * (i + 1) / nthreads, 0, 0, 0};
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
