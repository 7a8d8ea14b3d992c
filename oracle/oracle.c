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

/*
 * Conformer block-local attention with a relative-position term, in double precision.
 *
 * The pages (rullama 0.5.0, src/backend/dispatch/attention.rs,
 * block_local_attention_chained and its doc comment) give the call, not the kernel:
 * q_pad [padded_len, hidden] (Q projected and already per-dimension scaled),
 * k_padded / v_padded [(pad_left + padded_len + pad_right), hidden] (K with its scale
 * applied, zero padded), pos_proj [max_span, hidden] (sinusoidal relative positions
 * through a linear projection), chunk_size, context_size, max_span, max_past,
 * max_future, pad_left, logit_cap, head_dim 128, output [padded_len, hidden] of which
 * the caller keeps the first seq rows.  Readings of what they leave open:
 *   - hidden = H * D; head h owns columns [h D, (h + 1) D) of every row;
 *   - query row i sits at position i; row r of k_padded / v_padded holds position
 *     r - pad_left;
 *   - query i sees key position t iff i - max_past <= t <= i + max_future and
 *     0 <= t < seq (the zero padding outside [0, seq) is masked, not attended);
 *   - row j of pos_proj is the relative offset j - max_past (key minus query): row 0
 *     belongs to the key max_past positions before the query, row max_past to the
 *     query's own position, row max_span - 1 to the key max_future after it;
 *   - score s = q_i . k_t + q_i . pos_proj[t - i + max_past]; no further scale (the
 *     scale is folded into q_pad); if logit_cap > 0, s = cap * tanh(s / cap); 0 = off;
 *   - softmax over the visible keys, o_i = sum w v_t / sum w; a row with no visible key
 *     (a padding row far past seq) is written as zeros;
 *   - the geometry is consistent: max_span = max_past + max_future + 1,
 *     context_size = chunk_size + max_past + max_future, pad_left = max_past,
 *     padded_len a multiple of chunk_size, so the keys of every query of chunk c lie in
 *     the context rows [c chunk_size, c chunk_size + context_size) of k_padded.  Under
 *     this geometry the chunking changes which rows a kernel stages, never the result,
 *     so the definition below needs no chunk loop.
 *   q, o : [padded_len][H][D];  k, v : [kv_rows][H][D];  pos : [max_span][H][D]
 * Returns 0, or -1 on an argument error (an inconsistent geometry included).
 */
typedef struct {
    const double *q, *k, *v, *pos;
    double *o;
    int seq, padded_len, H, D, max_past, max_future, pad_left;
    double cap;
    long n_rows;
    long grab;
    long next;
    int workers;
    pthread_mutex_t mu;
} bl_job_t;

static void bl_row(const bl_job_t *J, int i, int h, double *score)
{
    const int D = J->D, H = J->H;
    const double *qrow = J->q + ((long)i * H + h) * D;
    double *orow = J->o + ((long)i * H + h) * D;
    const int span = J->max_past + J->max_future + 1;

    /* pass 1: scores of the visible keys t = i - max_past + j, j in [0, span) */
    double m = -INFINITY;
    int any = 0;
    for (int j = 0; j < span; ++j) {
        const long t = (long)i - J->max_past + j;
        if (t < 0 || t >= J->seq) { score[j] = NAN; continue; }
        const double *krow = J->k + ((t + J->pad_left) * H + h) * D;
        const double *prow = J->pos + ((long)j * H + h) * D;
        double content = 0.0, position = 0.0;
        for (int d = 0; d < D; ++d) {
            content += qrow[d] * krow[d];
            position += qrow[d] * prow[d];
        }
        double s = content + position;
        if (J->cap > 0.0) s = J->cap * tanh(s / J->cap);
        score[j] = s;
        if (s > m) m = s;
        any = 1;
    }
    for (int d = 0; d < D; ++d) orow[d] = 0.0;
    if (!any) return;

    /* pass 2: weights, their sum and the weighted sum of V rows */
    double l = 0.0;
    for (int j = 0; j < span; ++j) {
        if (isnan(score[j])) continue;
        const long t = (long)i - J->max_past + j;
        const double w = exp(score[j] - m);
        l += w;
        const double *vrow = J->v + ((t + J->pad_left) * H + h) * D;
        for (int d = 0; d < D; ++d) orow[d] += w * vrow[d];
    }
    for (int d = 0; d < D; ++d) orow[d] /= l;
}

static void *bl_worker(void *arg)
{
    bl_job_t *J = (bl_job_t *)arg;
    double *score = (double *)malloc(sizeof(double) * (size_t)(J->max_past + J->max_future + 1));
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
        for (long r = r0; r < r1; ++r) bl_row(J, (int)(r / J->H), (int)(r % J->H), score);
    }
    free(score);
    return NULL;
}

int oracle_block_local_f64(const double *q, const double *k, const double *v, const double *pos,
                           double *o, int seq, int padded_len, int kv_rows, int H, int D,
                           int chunk_size, int context_size, int max_span, int max_past,
                           int max_future, int pad_left, double logit_cap, int nthreads)
{
    if (H < 1 || D < 1 || chunk_size < 1 || seq < 1 || padded_len < seq) return -1;
    if (padded_len % chunk_size != 0 || max_past < 0 || max_future < 0) return -1;
    if (max_span != max_past + max_future + 1) return -1;
    if (context_size != chunk_size + max_past + max_future) return -1;
    if (pad_left != max_past || kv_rows < pad_left + seq) return -1;
    if (!(logit_cap >= 0.0)) return -1;
    bl_job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.pos = pos; J.o = o;
    J.seq = seq; J.padded_len = padded_len; J.H = H; J.D = D;
    J.max_past = max_past; J.max_future = max_future; J.pad_left = pad_left;
    J.cap = logit_cap;
    J.n_rows = (long)padded_len * H;
    pthread_mutex_init(&J.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    J.grab = J.n_rows / (4L * nthreads);
    if (J.grab < 1) J.grab = 1;
    if (J.grab > 64) J.grab = 64;
    pthread_t th[256];
    int started = 0;
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&th[started], NULL, bl_worker, &J) == 0) ++started;
    bl_worker(&J);
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    pthread_mutex_destroy(&J.mu);
    g_threads_used = J.workers;
    return 0;
}
