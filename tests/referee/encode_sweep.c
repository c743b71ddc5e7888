/*
 * Brute-force referee for an FP8 encoder, used to pin the oracle's encoder over
 * every fp32 bit pattern.  It shares nothing with the oracle: it receives the
 * 256 decoded values of the format from the caller (the test takes them from
 * torch's float8 dtypes), sorts the finite non-negative ones, and for each
 * input picks the nearest value, ties to the even code, magnitudes above the
 * largest finite value saturating to it.  The encoder under test is called
 * through a function pointer.  Build: gcc -O2 -pthread -shared -fPIC.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef uint8_t (*encoder_fn)(int fmt, float x);

typedef struct { double value; int code; } entry;

typedef struct {
    const entry *tab;
    int ntab;
    encoder_fn enc;
    int fmt;
    uint64_t lo, hi;         /* bit patterns [lo, hi) */
    uint64_t mismatches;
    uint64_t first_bad;      /* first mismatching bit pattern, or ~0 */
    int first_got, first_want;
} job;

static int cmp_entry(const void *a, const void *b)
{
    double x = ((const entry *)a)->value, y = ((const entry *)b)->value;
    return x < y ? -1 : x > y ? 1 : 0;
}

static int referee_code(const entry *tab, int ntab, float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    int sign = (int)(u >> 31) << 7;
    double a = fabs((double)x);
    if (a >= tab[ntab - 1].value) return sign | tab[ntab - 1].code; /* saturate */
    /* largest i with tab[i].value <= a (tab[0] is zero) */
    int lo = 0, hi = ntab - 1;
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (tab[mid].value <= a) lo = mid; else hi = mid;
    }
    double dlo = a - tab[lo].value, dhi = tab[hi].value - a; /* exact in double */
    int pick;
    if (dlo < dhi) pick = tab[lo].code;
    else if (dhi < dlo) pick = tab[hi].code;
    else pick = (tab[lo].code & 1) == 0 ? tab[lo].code : tab[hi].code;
    return sign | pick;
}

static void *run(void *arg)
{
    job *j = (job *)arg;
    for (uint64_t b = j->lo; b < j->hi; b++) {
        uint32_t u = (uint32_t)b;
        float x;
        memcpy(&x, &u, 4);
        if (isnan(x)) continue; /* NaN input is outside the contract */
        int want = referee_code(j->tab, j->ntab, x);
        int got = j->enc(j->fmt, x);
        if (got != want) {
            if (j->mismatches == 0) {
                j->first_bad = b;
                j->first_got = got;
                j->first_want = want;
            }
            j->mismatches++;
        }
    }
    return NULL;
}

/*
 * values: the 256 decoded values of the format (NaN/Inf entries are ignored).
 * Sweeps bit patterns [lo, hi) with nthreads threads.  Returns the number of
 * mismatches; *first_bad / *got / *want describe the first one found.
 */
uint64_t sweep_encoder(const double *values, uintptr_t encoder, int fmt, uint64_t lo,
                       uint64_t hi, int nthreads, uint64_t *first_bad, int *got, int *want)
{
    entry tab[256];
    int ntab = 0;
    for (int c = 0; c < 128; c++) {
        if (!isfinite(values[c]) || signbit(values[c])) continue;
        tab[ntab].value = values[c];
        tab[ntab].code = c;
        ntab++;
    }
    qsort(tab, (size_t)ntab, sizeof(entry), cmp_entry);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 64) nthreads = 64;
    job jobs[64];
    pthread_t th[64];
    uint64_t span = (hi - lo + (uint64_t)nthreads - 1) / (uint64_t)nthreads;
    for (int t = 0; t < nthreads; t++) {
        jobs[t].tab = tab;
        jobs[t].ntab = ntab;
        jobs[t].enc = (encoder_fn)encoder;
        jobs[t].fmt = fmt;
        jobs[t].lo = lo + span * (uint64_t)t;
        jobs[t].hi = jobs[t].lo + span < hi ? jobs[t].lo + span : hi;
        if (jobs[t].lo > hi) jobs[t].lo = hi;
        jobs[t].mismatches = 0;
        jobs[t].first_bad = ~(uint64_t)0;
        pthread_create(&th[t], NULL, run, &jobs[t]);
    }
    uint64_t total = 0;
    *first_bad = ~(uint64_t)0;
    for (int t = 0; t < nthreads; t++) {
        pthread_join(th[t], NULL);
        total += jobs[t].mismatches;
        if (jobs[t].mismatches && jobs[t].first_bad < *first_bad) {
            *first_bad = jobs[t].first_bad;
            *got = jobs[t].first_got;
            *want = jobs[t].first_want;
        }
    }
    return total;
}
