/*
 * Seeded synthetic inputs: SplitMix64 uniforms and Box-Muller normals, threaded.
 * Holds no attention arithmetic.  The generator definition is in synth/__init__.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>

static inline uint64_t mix64(uint64_t z)
{
    z ^= z >> 30; z *= 0xBF58476D1CE4E5B9ULL;
    z ^= z >> 27; z *= 0x94D049BB133111EBULL;
    z ^= z >> 31;
    return z;
}

/* output i (0-based) of stream `seed` */
static inline uint64_t sm64(uint64_t seed, uint64_t i)
{
    return mix64(seed + (i + 1) * 0x9E3779B97F4A7C15ULL);
}

static inline double u01(uint64_t x) { return (double)(x >> 11) * (1.0 / 9007199254740992.0); }

void synth_uniform(uint64_t seed, uint64_t start, uint64_t n, double *out)
{
    for (uint64_t i = 0; i < n; ++i) out[i] = u01(sm64(seed, start + i));
}

typedef struct { uint64_t seed, start, n; float *out; } job_t;

/* normal number k of the stream: pair k/2 from uniforms (k & ~1, k | 1) */
static void *normal_worker(void *arg)
{
    job_t *J = (job_t *)arg;
    const double two_pi = 6.283185307179586476925286766559;
    for (uint64_t i = 0; i < J->n; ++i) {
        const uint64_t k = J->start + i;
        const uint64_t p = k >> 1;
        const double ua = u01(sm64(J->seed, 2 * p));
        const double ub = u01(sm64(J->seed, 2 * p + 1));
        const double r = sqrt(-2.0 * log1p(-ua));
        const double th = two_pi * ub;
        J->out[i] = (float)((k & 1) ? r * sin(th) : r * cos(th));
    }
    return 0;
}

/* n standard normals (rounded to float32) with stream indices start .. start+n-1 */
void synth_normal_f32(uint64_t seed, uint64_t start, uint64_t n, float *out, int threads)
{
    if (threads < 1) threads = 1;
    if (threads > 64) threads = 64;
    if (n < 65536) threads = 1;
    job_t jobs[64];
    pthread_t th[64];
    int created[64] = {0};
    const uint64_t per = (n + threads - 1) / threads;
    for (int t = 0; t < threads; ++t) {
        const uint64_t lo = per * t;
        if (lo >= n) break;
        jobs[t].seed = seed;
        jobs[t].start = start + lo;
        jobs[t].n = (lo + per > n ? n : lo + per) - lo;
        jobs[t].out = out + lo;
        if (t == 0) continue;
        if (pthread_create(&th[t], 0, normal_worker, &jobs[t]) == 0) created[t] = 1;
        else normal_worker(&jobs[t]);
    }
    normal_worker(&jobs[0]);
    for (int t = 1; t < threads; ++t)
        if (created[t]) pthread_join(th[t], 0);
}
