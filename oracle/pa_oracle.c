/*
 * pa_oracle.c -- fp64 CPU oracle for the paged-attention decode step.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It is plain and slow on
 * purpose and shares no code, header or constant with the HIP library.
 *
 * What it computes (the definition the GPU path must reach):
 *   For each sequence b and query head h
 *     kvh = h / (H / Hkv)                      -- grouped-query head mapping,
 *        benchmark_decoding.py, kernels and reference_output (h // groups).
 *     live tokens t < context_lens[b] whose block-table entry
 *        blk = block_tables[b][t / block_size] is not -1; their rows are
 *        K_t = k_cache[blk][t % block_size][kvh][:], V_t likewise
 *        -- "Decoding Benchmark" docs page, "What paged attention decode does"
 *        (lookup pattern) and "Block table lookup mechanics" (-1 = unallocated).
 *     s_t = scale * sum_i q[b][h][i] * K_t[i]
 *     out[b][h] = sum_t softmax(s)_t * V_t
 *        -- benchmark_decoding.py, reference_output: softmax of the scaled
 *        scores times the gathered V rows.
 *
 * Readings where the pages are silent or disagree:
 *   - a -1 entry inside the context removes those tokens from the softmax
 *     (the Triton (new) kernel's valid mask; the docs page: -1 = not
 *     allocated);
 *   - an empty live set (context_len 0, or every block -1) gives zeros (the
 *     gather-then-softmax reference yields an empty sum);
 *   - context_len above max_blocks * block_size, a table entry below -1 or at
 *     or past the pool size are rejected as invalid input.
 *
 * Three entry points compute the same result by different routes; the test
 * suite checks that they agree and pins the first against library routines,
 * closed forms and invariants:
 *   pa_oracle_decode        gather, then dense two-pass softmax (the definition)
 *   pa_oracle_decode_online one pass over tiles with a running max and
 *                           normaliser (Triton kernels of benchmark_decoding.py;
 *                           docs page, "Why CUDA chunk processing matters")
 *   pa_oracle_decode_split  Flash-Decoding: per-partition local statistics
 *                           (max, sum, weighted values) merged afterwards
 *                           (flash-decoding-bench design note, implementations)
 *
 * Inputs are float32 arrays (bf16 inputs arrive already widened, exactly);
 * every arithmetic step runs in double.  Output is double [B][H][d].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_ERR_NULL (-1)
#define OR_ERR_SHAPE (-2)
#define OR_ERR_CONTEXT (-3)
#define OR_ERR_TABLE (-4)
#define OR_ERR_NOMEM (-5)

typedef struct {
    const float *q, *k, *v;
    const int32_t *table, *lens;
    int B, H, Hkv, d, bs, max_blocks;
    long long pool;
    double scale;
} problem_t;

static int check(const problem_t *p, double *out) {
    if (!out || !p->q || !p->k || !p->v || !p->table || !p->lens) return OR_ERR_NULL;
    if (p->B < 0 || p->H <= 0 || p->Hkv <= 0 || p->d <= 0 || p->bs <= 0 || p->max_blocks <= 0)
        return OR_ERR_SHAPE;
    if (p->H % p->Hkv != 0) return OR_ERR_SHAPE;
    for (int b = 0; b < p->B; ++b) {
        int n = p->lens[b];
        if (n < 0 || (long long)n > (long long)p->max_blocks * p->bs) return OR_ERR_CONTEXT;
        for (int j = 0; j < p->max_blocks; ++j) {
            int32_t blk = p->table[(size_t)b * p->max_blocks + j];
            if (blk < -1 || (long long)blk >= p->pool) return OR_ERR_TABLE;
        }
    }
    return OR_OK;
}

/* Address of element 0 of row (blk, slot, kvh) in a [pool][bs][Hkv][d] cache. */
static const float *row(const problem_t *p, const float *cache, int32_t blk, int slot, int kvh) {
    size_t off = (((size_t)blk * p->bs + slot) * p->Hkv + kvh) * (size_t)p->d;
    return cache + off;
}

/* Gather the live tokens of sequence b in logical order: fills toks[] with
 * token indices t and returns their count. */
static int live_tokens(const problem_t *p, int b, int *toks) {
    int n = p->lens[b], count = 0;
    for (int t = 0; t < n; ++t) {
        int32_t blk = p->table[(size_t)b * p->max_blocks + t / p->bs];
        if (blk == -1) continue;
        toks[count++] = t;
    }
    return count;
}

static double score(const problem_t *p, int b, int h, int kvh, int t) {
    int32_t blk = p->table[(size_t)b * p->max_blocks + t / p->bs];
    const float *kr = row(p, p->k, blk, t % p->bs, kvh);
    const float *qr = p->q + ((size_t)b * p->H + h) * p->d;
    double dot = 0.0;
    for (int i = 0; i < p->d; ++i) dot += (double)qr[i] * (double)kr[i];
    return p->scale * dot;
}

static const float *vrow(const problem_t *p, int b, int kvh, int t) {
    int32_t blk = p->table[(size_t)b * p->max_blocks + t / p->bs];
    return row(p, p->v, blk, t % p->bs, kvh);
}

/* ---- definition: gather, then two-pass softmax ------------------------------ */
static void head_two_pass(const problem_t *p, int b, int h, const int *toks, int n,
                          double *s, double *o) {
    int kvh = h / (p->H / p->Hkv);
    for (int i = 0; i < p->d; ++i) o[i] = 0.0;
    if (n == 0) return;
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
        s[j] = score(p, b, h, kvh, toks[j]);
        if (s[j] > m) m = s[j];
    }
    double z = 0.0;
    for (int j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        z += s[j];
    }
    for (int j = 0; j < n; ++j) {
        const float *vr = vrow(p, b, kvh, toks[j]);
        double w = s[j] / z;
        for (int i = 0; i < p->d; ++i) o[i] += w * (double)vr[i];
    }
}

/* ---- one pass: running max m_i and normaliser l_i over tiles ---------------- */
static void head_online(const problem_t *p, int b, int h, int tile, double *s, double *o) {
    int kvh = h / (p->H / p->Hkv);
    int n = p->lens[b];
    double m_i = -INFINITY, l_i = 0.0;
    for (int i = 0; i < p->d; ++i) o[i] = 0.0; /* o holds acc */
    for (int start = 0; start < n; start += tile) {
        int end = start + tile < n ? start + tile : n;
        int live = 0;
        double m_ij = -INFINITY;
        for (int t = start; t < end; ++t) {
            int32_t blk = p->table[(size_t)b * p->max_blocks + t / p->bs];
            if (blk == -1) { s[t - start] = NAN; continue; }
            s[t - start] = score(p, b, h, kvh, t);
            if (s[t - start] > m_ij) m_ij = s[t - start];
            ++live;
        }
        if (live == 0) continue;
        double m_new = m_i > m_ij ? m_i : m_ij;
        double alpha = exp(m_i - m_new); /* exp(-inf) = 0 on the first live tile */
        for (int i = 0; i < p->d; ++i) o[i] *= alpha;
        l_i *= alpha;
        for (int t = start; t < end; ++t) {
            if (isnan(s[t - start])) continue;
            double pt = exp(s[t - start] - m_new);
            const float *vr = vrow(p, b, kvh, t);
            for (int i = 0; i < p->d; ++i) o[i] += pt * (double)vr[i];
            l_i += pt;
        }
        m_i = m_new;
    }
    if (l_i > 0.0)
        for (int i = 0; i < p->d; ++i) o[i] /= l_i;
}

/* ---- split: per-partition (max, sum, weighted values), then merge ----------- */
static void head_split(const problem_t *p, int b, int h, int parts, double *s,
                       double *acc_p, double *o) {
    int kvh = h / (p->H / p->Hkv);
    int n = p->lens[b];
    int bpp = (p->max_blocks + parts - 1) / parts;
    double *m_p = s;                 /* parts entries */
    double *l_p = s + parts;         /* parts entries */
    for (int q = 0; q < parts; ++q) {
        double *a = acc_p + (size_t)q * p->d;
        for (int i = 0; i < p->d; ++i) a[i] = 0.0;
        m_p[q] = -INFINITY;
        l_p[q] = 0.0;
        int t0 = q * bpp * p->bs, t1 = (q + 1) * bpp * p->bs;
        if (t1 > n) t1 = n;
        /* local max over the partition's live tokens */
        for (int t = t0; t < t1; ++t) {
            if (p->table[(size_t)b * p->max_blocks + t / p->bs] == -1) continue;
            double st = score(p, b, h, kvh, t);
            if (st > m_p[q]) m_p[q] = st;
        }
        if (m_p[q] == -INFINITY) continue; /* empty partition: l_p = 0 */
        for (int t = t0; t < t1; ++t) {
            if (p->table[(size_t)b * p->max_blocks + t / p->bs] == -1) continue;
            double w = exp(score(p, b, h, kvh, t) - m_p[q]);
            const float *vr = vrow(p, b, kvh, t);
            for (int i = 0; i < p->d; ++i) a[i] += w * (double)vr[i];
            l_p[q] += w;
        }
    }
    /* merge: rescale every partition to the global max and sum */
    double M = -INFINITY;
    for (int q = 0; q < parts; ++q)
        if (l_p[q] > 0.0 && m_p[q] > M) M = m_p[q];
    for (int i = 0; i < p->d; ++i) o[i] = 0.0;
    if (M == -INFINITY) return;
    double L = 0.0;
    for (int q = 0; q < parts; ++q) {
        if (l_p[q] == 0.0) continue;
        double f = exp(m_p[q] - M);
        L += l_p[q] * f;
        const double *a = acc_p + (size_t)q * p->d;
        for (int i = 0; i < p->d; ++i) o[i] += a[i] * f;
    }
    for (int i = 0; i < p->d; ++i) o[i] /= L;
}

enum { MODE_TWO_PASS = 0, MODE_ONLINE = 1, MODE_SPLIT = 2 };

static int run(const problem_t *p, double *out, int mode, int param, int threads) {
    int rc = check(p, out);
    if (rc != OR_OK) return rc;
    if ((mode == MODE_ONLINE || mode == MODE_SPLIT) && param <= 0) return OR_ERR_SHAPE;
    if (p->B == 0) return OR_OK;
    int cap = p->max_blocks * p->bs;
    int pairs = p->B * p->H;
    int failed = 0;
#ifdef _OPENMP
    if (threads <= 0) threads = omp_get_max_threads();
#pragma omp parallel num_threads(threads)
#endif
    {
        size_t ns = (size_t)cap + 2 * (size_t)(param > 0 ? param : 1) + 1;
        double *s = (double *)malloc(ns * sizeof(double));
        int *toks = (int *)malloc(((size_t)cap + 1) * sizeof(int));
        double *acc_p = mode == MODE_SPLIT
            ? (double *)malloc((size_t)param * p->d * sizeof(double)) : NULL;
        int ok = s && toks && (mode != MODE_SPLIT || acc_p);
        if (!ok) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic)
#endif
        for (int pair = 0; pair < pairs; ++pair) {
            if (!ok) continue;
            int b = pair / p->H, h = pair % p->H;
            double *o = out + (size_t)pair * p->d;
            if (mode == MODE_TWO_PASS) {
                int n = live_tokens(p, b, toks);
                head_two_pass(p, b, h, toks, n, s, o);
            } else if (mode == MODE_ONLINE) {
                head_online(p, b, h, param, s, o);
            } else {
                head_split(p, b, h, param, s, acc_p, o);
            }
        }
        free(s);
        free(toks);
        free(acc_p);
    }
    return failed ? OR_ERR_NOMEM : OR_OK;
}

#define PROBLEM                                                                       \
    problem_t p = {q, k_cache, v_cache, block_tables, context_lens, B, H, Hkv, d,     \
                   block_size, max_blocks, num_pool_blocks, scale}

int pa_oracle_decode(double *out, const float *q, const float *k_cache, const float *v_cache,
                     const int32_t *block_tables, const int32_t *context_lens, int B, int H,
                     int Hkv, int d, int block_size, int max_blocks, long long num_pool_blocks,
                     double scale, int num_threads) {
    PROBLEM;
    return run(&p, out, MODE_TWO_PASS, 0, num_threads);
}

int pa_oracle_decode_online(double *out, const float *q, const float *k_cache,
                            const float *v_cache, const int32_t *block_tables,
                            const int32_t *context_lens, int B, int H, int Hkv, int d,
                            int block_size, int max_blocks, long long num_pool_blocks,
                            double scale, int tile, int num_threads) {
    PROBLEM;
    return run(&p, out, MODE_ONLINE, tile, num_threads);
}

int pa_oracle_decode_split(double *out, const float *q, const float *k_cache,
                           const float *v_cache, const int32_t *block_tables,
                           const int32_t *context_lens, int B, int H, int Hkv, int d,
                           int block_size, int max_blocks, long long num_pool_blocks,
                           double scale, int num_partitions, int num_threads) {
    PROBLEM;
    return run(&p, out, MODE_SPLIT, num_partitions, num_threads);
}

int pa_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
