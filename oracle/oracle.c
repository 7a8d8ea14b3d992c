/*
 * Reference semantics of softmax attention, in double precision, on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no code, header, table or helper with the HIP library.
 *
 * What it computes is the plain definition of scaled dot-product attention.
 * Flash attention (online softmax over K/V tiles, as described for the
 * vision flash kernels in rullama 0.5.0 src/backend/dispatch/attention.rs,
 * vision_attention_flash_chained) reaches the same value up to rounding
 * order, so the oracle materialises every score row in full and makes two
 * passes over it (max, then exp/sum/weighted V).  No tiling, no rescaling.
 *
 * Problem statement (doppler gpu/kernels/attention.js, 0.1.9->0.2.0,
 * createAttentionUniformBuffer and executeAttention): numHeads, numKVHeads,
 * headDim, kvLen, seqLen, scale, causal, startPos, attnSoftcap,
 * slidingWindow.  Readings of points the pages leave open:
 *   - query head h reads KV head floor(h / (H / Hkv))  (contiguous groups);
 *   - query row i of a block of S rows sits at absolute position
 *     p_i = kv_len - S + i (doppler run.js 0.1.0: startPos = currentSeqLen,
 *     kvLen = currentSeqLen + numTokens);
 *   - key j is visible iff j < kv_len, (!causal || j <= p_i) and
 *     (window == 0 || p_i - j < window): the window holds `window` keys
 *     including the query's own position (doppler run.js clips kvLen to the
 *     window and sets kvStart = total - kvLen);
 *   - the logit softcap c > 0 maps the scaled score s to c * tanh(s / c)
 *     (attnSoftcap, "0 = disabled"); 0 disables it;
 *   - a row that sees no key (out of contract) is written as zeros.
 *
 * Built with plain gcc -O2, no -ffast-math.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v;
    double *o;
    int B, S, Lmax, H, Hkv, D;
    const int *kv_len;
    int causal, window;
    double softcap, scale;
    long n_rows;          /* B * S * H */
    long grab;            /* rows taken per visit of the work counter */
    long next;            /* shared work counter, guarded by mu */
    int workers;          /* threads that computed at least one row, guarded by mu */
    pthread_mutex_t mu;
} job_t;

/* Threads that computed at least one row in the last oracle_attention_f64 call of the
 * process (a figure for reports; not synchronised between concurrent calls). */
static int g_threads_used = 0;

/* One output row: batch b, query row i, query head h. */
static void one_row(const job_t *J, int b, int i, int h, double *score)
{
    const int G = J->H / J->Hkv;
    const int kvh = h / G;
    const int L = J->kv_len[b];
    const long p = (long)L - J->S + i;
    const double *qrow = J->q + (((long)b * J->S + i) * J->H + h) * J->D;
    double *orow = J->o + (((long)b * J->S + i) * J->H + h) * J->D;

    /* pass 1: scores of visible keys, and their maximum */
    double m = -INFINITY;
    int any = 0;
    for (long j = 0; j < L; ++j) {
        int visible = 1;
        if (J->causal && j > p) visible = 0;
        if (J->window > 0 && p - j >= J->window) visible = 0;
        if (!visible) { score[j] = NAN; continue; }
        const double *krow = J->k + (((long)b * J->Lmax + j) * J->Hkv + kvh) * J->D;
        double dot = 0.0;
        for (int d = 0; d < J->D; ++d) dot += qrow[d] * krow[d];
        double s = J->scale * dot;
        if (J->softcap > 0.0) s = J->softcap * tanh(s / J->softcap);
        score[j] = s;
        if (s > m) m = s;
        any = 1;
    }
    for (int d = 0; d < J->D; ++d) orow[d] = 0.0;
    if (!any) return;

    /* pass 2: weights, their sum, and the weighted sum of V rows */
    double l = 0.0;
    for (long j = 0; j < L; ++j) {
        if (isnan(score[j])) continue;
        const double w = exp(score[j] - m);
        l += w;
        const double *vrow = J->v + (((long)b * J->Lmax + j) * J->Hkv + kvh) * J->D;
        for (int d = 0; d < J->D; ++d) orow[d] += w * vrow[d];
    }
    for (int d = 0; d < J->D; ++d) orow[d] /= l;
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    double *score = (double *)malloc(sizeof(double) * (size_t)(J->Lmax > 0 ? J->Lmax : 1));
    if (!score) return NULL;
    int counted = 0;
    for (;;) {
        long r0;
        pthread_mutex_lock(&J->mu);
        r0 = J->next;
        J->next += J->grab;
        if (r0 < J->n_rows && !counted) {
            counted = 1;
            J->workers += 1;
        }
        pthread_mutex_unlock(&J->mu);
        if (r0 >= J->n_rows) break;
        long r1 = r0 + J->grab < J->n_rows ? r0 + J->grab : J->n_rows;
        for (long r = r0; r < r1; ++r) {
            const int h = (int)(r % J->H);
            const int i = (int)((r / J->H) % J->S);
            const int b = (int)(r / ((long)J->H * J->S));
            one_row(J, b, i, h, score);
        }
    }
    free(score);
    return NULL;
}

/*
 * Softmax attention over canonical double arrays.
 *   q, o : [B][S][H][D]
 *   k, v : [B][Lmax][Hkv][D]   (rows j >= kv_len[b] are never read)
 *   kv_len : [B], 1 <= kv_len[b] <= Lmax, and kv_len[b] >= S
 * Returns 0, or -1 on an argument error.  nthreads <= 0 means 1.
 */
int oracle_attention_f64(const double *q, const double *k, const double *v, double *o,
                         int B, int S, int Lmax, const int *kv_len, int H, int Hkv, int D,
                         int causal, int window, double softcap, double scale, int nthreads)
{
    if (B < 1 || S < 1 || Lmax < 1 || H < 1 || Hkv < 1 || D < 1 || H % Hkv != 0) return -1;
    if (window < 0 || !(softcap >= 0.0) || !isfinite(scale)) return -1;
    for (int b = 0; b < B; ++b)
        if (kv_len[b] < S || kv_len[b] > Lmax) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.o = o;
    J.B = B; J.S = S; J.Lmax = Lmax; J.H = H; J.Hkv = Hkv; J.D = D;
    J.kv_len = kv_len; J.causal = causal; J.window = window;
    J.softcap = softcap; J.scale = scale;
    J.n_rows = (long)B * S * H;
    J.next = 0;
    J.workers = 0;
    pthread_mutex_init(&J.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    /* about four grabs per thread, at most 16 rows each, so that a call with few (long)
     * rows, such as one decode token over 32 heads, still spreads over every thread */
    J.grab = J.n_rows / (4L * nthreads);
    if (J.grab < 1) J.grab = 1;
    if (J.grab > 16) J.grab = 16;
    pthread_t th[256];
    int started = 0;
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&th[started], NULL, worker, &J) == 0) ++started;
    worker(&J);
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    pthread_mutex_destroy(&J.mu);
    g_threads_used = J.workers;
    return 0;
}

int oracle_threads_used(void) { return g_threads_used; }

/*
 * Dequantisation of a symmetric int8 cache row: x = q8 * scale, one f32 scale
 * per (token, kv head) row of D values.  The int8 cold tier of doppler
 * (executeAttentionTieredQuant: packed K/V plus separate K and V scale
 * buffers, f32 Q required) gives the format; the per-row granularity is the
 * reading adopted.  The product of an int8 and an f32 is exact in double.
 */
void oracle_dequant_i8(const int8_t *q8, const float *scale, long rows, int D, double *out)
{
    for (long r = 0; r < rows; ++r)
        for (int d = 0; d < D; ++d)
            out[r * D + d] = (double)q8[r * D + d] * (double)scale[r];
}
