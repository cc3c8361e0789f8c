/*
 * synth.c -- seeded synthetic inputs (weights, codes, scales).
 *
 * This is input generation only: it holds none of the coder's or the
 * dequantiser's arithmetic. Both the CPU oracle's tests and the GPU path's
 * tests and benchmark draw their inputs from here.
 *
 * Every value is a pure function of (key, index): a counter-based generator,
 * so any slice of a tensor can be produced by any thread, in any order, with
 * the same result. The generator is SplitMix64 (Steele, Lea, Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014) used in counter
 * mode: output i of stream `key` is mix64(key + (i + 1) * 0x9E3779B97F4A7C15),
 * where mix64 is that paper's output function.
 *
 * Integer codes are drawn by inverse-CDF lookup: the caller passes the 254
 * cumulative thresholds of a distribution over the integers -127..127 (as
 * fractions of 2^64), and the code is -127 plus the number of thresholds at
 * or below the 64-bit draw. This samples the rounded-and-clipped distribution
 * exactly, with integer operations only.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t key, uint64_t i)
{
    return mix64(key + (i + 1u) * 0x9E3779B97F4A7C15ull);
}

uint64_t syn_mix64(uint64_t z) { return mix64(z); }
uint64_t syn_draw(uint64_t key, uint64_t i) { return draw(key, i); }

/* ---- thread fan-out ---- */

typedef struct {
    int what;
    uint64_t key, begin, end;
    const uint64_t *thr;
    const uint8_t *start;
    double a, b;
    void *out;
} job_t;

/* uniform double in [0, 1) from the top 53 bits */
static inline double unit53(uint64_t u) { return (double)(u >> 11) * (1.0 / 9007199254740992.0); }

static void run_range(job_t *j)
{
    if (j->what == 0) { /* int8 codes by inverse CDF */
        int8_t *o = (int8_t *)j->out;
        const uint64_t *t = j->thr;
        const uint8_t *start = j->start;
        for (uint64_t i = j->begin; i < j->end; i++) {
            uint64_t u = draw(j->key, i);
            /* number of thresholds <= u: start from the count at the bottom
             * of u's 2^48-wide bucket and step over the few inside it */
            unsigned k = start[u >> 48];
            while (k < 254u && t[k] <= u)
                k++;
            o[i] = (int8_t)((int)k - 127);
        }
    } else if (j->what == 1) { /* normal(0, sigma) as fp32, Box-Muller */
        float *o = (float *)j->out;
        for (uint64_t i = j->begin; i < j->end; i++) {
            uint64_t u1 = draw(j->key, 2u * i), u2 = draw(j->key, 2u * i + 1u);
            double r1 = 1.0 - unit53(u1); /* (0, 1] */
            double r2 = unit53(u2);
            double z = sqrt(-2.0 * log(r1)) * cos(6.283185307179586 * r2);
            o[i] = (float)(j->a * z);
        }
    } else { /* uniform [a, b) as fp32 */
        float *o = (float *)j->out;
        for (uint64_t i = j->begin; i < j->end; i++)
            o[i] = (float)(j->a + (j->b - j->a) * unit53(draw(j->key, i)));
    }
}

static void *worker(void *p)
{
    run_range((job_t *)p);
    return NULL;
}

static void fan_out(job_t base, uint64_t n, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 64)
        nthreads = 64;
    if ((uint64_t)nthreads > n / 65536 + 1)
        nthreads = (int)(n / 65536 + 1);
    pthread_t th[64];
    job_t jobs[64];
    for (int t = 0; t < nthreads; t++) {
        jobs[t] = base;
        jobs[t].begin = n * (uint64_t)t / (uint64_t)nthreads;
        jobs[t].end = n * (uint64_t)(t + 1) / (uint64_t)nthreads;
    }
    for (int t = 1; t < nthreads; t++)
        pthread_create(&th[t], NULL, worker, &jobs[t]);
    run_range(&jobs[0]);
    for (int t = 1; t < nthreads; t++)
        pthread_join(th[t], NULL);
}

/* thr: 254 ascending thresholds (entries past 253 are ignored). */
void syn_codes_int8(uint64_t key, const uint64_t *thr, uint64_t n, int8_t *out, int nthreads)
{
    uint8_t *start = (uint8_t *)malloc(65536);
    for (uint64_t b = 0; b < 65536; b++) {
        unsigned k = 0;
        while (k < 254u && thr[k] <= (b << 48))
            k++;
        start[b] = (uint8_t)k;
    }
    job_t j = {0, key, 0, 0, thr, start, 0, 0, out};
    fan_out(j, n, nthreads);
    free(start);
}

void syn_normal_f32(uint64_t key, double sigma, uint64_t n, float *out, int nthreads)
{
    job_t j = {1, key, 0, 0, NULL, NULL, sigma, 0, out};
    fan_out(j, n, nthreads);
}

void syn_uniform_f32(uint64_t key, double lo, double hi, uint64_t n, float *out, int nthreads)
{
    job_t j = {2, key, 0, 0, NULL, NULL, lo, hi, out};
    fan_out(j, n, nthreads);
}
