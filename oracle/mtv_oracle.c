/*
 * CPU oracle for absorbed-MLA tree-verify attention (see mtv_oracle.h).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path.
 *
 * The steps follow the order the problem is stated in: gather the sequence's
 * latent rows through the per-token page table, score every key against the
 * query, drop the tree keys the node may not see, normalise with a softmax and
 * take the weighted sum of the 512-d latents. Each step is written as its plain
 * definition; the only parallelism is over independent output rows.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared -pthread
 */
#define _POSIX_C_SOURCE 200809L
#include "mtv_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define D_QK 576
#define D_V 512

/* ------------------------------------------------------------------ bf16 */

double mtv_oracle_bf16_to_f64(uint16_t x)
{
    /* bf16 is the upper half of an IEEE binary32: widening is exact. */
    uint32_t u = (uint32_t)x << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

uint16_t mtv_oracle_f64_to_bf16(double x)
{
    /* IEEE-754 round-to-nearest, ties-to-even, from double straight to bf16
     * (8 significant bits, binary32 exponent range), no intermediate float. */
    const uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(x);
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0)
        return sign;
    int e;
    (void)frexp(a, &e);          /* a in [2^(e-1), 2^e) */
    int ulp_exp = e - 8;         /* spacing of bf16 values in that binade */
    if (ulp_exp < -133)          /* below 2^-126 the spacing stays 2^-133 */
        ulp_exp = -133;
    double units = ldexp(a, -ulp_exp);   /* exact: scaling by a power of two */
    double r = nearbyint(units);         /* default mode: nearest, ties to even */
    double v = ldexp(r, ulp_exp);
    if (v >= 0x1p128)
        return (uint16_t)(sign | 0x7F80u);   /* overflow rounds to infinity */
    float f = (float)v;                       /* exact: v is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

/* ------------------------------------------------------------ per-row work */

typedef struct {
    int N, H, W, S;
    int64_t b;
    const uint16_t* q;          /* whole q */
    const double* K;            /* gathered rows of sequence b: [S][576] */
    const uint32_t* tree_mask;  /* whole mask */
    double scale;
    const int64_t* rows;        /* rows of sequence b to compute */
    int64_t nrows;
    uint16_t* out_bf16;
    float* lse_f32;
    double* out_f64;
    double* lse_f64;
    int tid, nthreads;
    int err;
} row_job;

/* Whether tree node i of sequence b may attend key position p (p < S). */
static int key_visible(const row_job* J, int i, int p)
{
    int prefix = J->S - J->N;
    if (p < prefix)
        return 1;                                /* the prefix needs no mask */
    int j = p - prefix;                          /* tree node held at position p */
    const uint32_t* words = J->tree_mask + ((J->b * J->N + i) * (int64_t)J->W);
    return (int)((words[j >> 5] >> (j & 31)) & 1u);
}

static void one_row(const row_job* J, int64_t r, double* qd, double* s, unsigned char* vis, double* acc)
{
    const int64_t per_seq = (int64_t)J->N * J->H;
    const int i = (int)((r % per_seq) / J->H);   /* tree node of this row */
    const int S = J->S;

    for (int d = 0; d < D_QK; ++d)
        qd[d] = mtv_oracle_bf16_to_f64(J->q[r * D_QK + d]);

    /* scores and visibility */
    int any = 0;
    double m = -INFINITY;
    for (int p = 0; p < S; ++p) {
        vis[p] = (unsigned char)key_visible(J, i, p);
        if (!vis[p])
            continue;
        const double* k = J->K + (int64_t)p * D_QK;
        double dot = 0.0;
        for (int d = 0; d < D_QK; ++d)
            dot += qd[d] * k[d];
        s[p] = J->scale * dot;
        if (!any || s[p] > m)
            m = s[p];
        any = 1;
    }

    double lse;
    for (int c = 0; c < D_V; ++c)
        acc[c] = 0.0;
    if (!any) {
        lse = -INFINITY;                         /* empty visible set: out = 0 */
    } else {
        /* softmax normaliser and weighted latent sum */
        double l = 0.0;
        for (int p = 0; p < S; ++p) {
            if (!vis[p])
                continue;
            double e = exp(s[p] - m);
            l += e;
            const double* v = J->K + (int64_t)p * D_QK;
            for (int c = 0; c < D_V; ++c)
                acc[c] += e * v[c];
        }
        for (int c = 0; c < D_V; ++c)
            acc[c] = acc[c] / l;
        lse = m + log(l);
    }

    for (int c = 0; c < D_V; ++c) {
        J->out_bf16[r * D_V + c] = mtv_oracle_f64_to_bf16(acc[c]);
        if (J->out_f64)
            J->out_f64[r * D_V + c] = acc[c];
    }
    J->lse_f32[r] = (float)lse;
    if (J->lse_f64)
        J->lse_f64[r] = lse;
}

static void* row_worker(void* arg)
{
    row_job* J = (row_job*)arg;
    double* qd = (double*)malloc(sizeof(double) * D_QK);
    double* acc = (double*)malloc(sizeof(double) * D_V);
    double* s = (double*)malloc(sizeof(double) * (size_t)(J->S > 0 ? J->S : 1));
    unsigned char* vis = (unsigned char*)malloc((size_t)(J->S > 0 ? J->S : 1));
    if (!qd || !acc || !s || !vis) {
        J->err = MTV_ORACLE_ERR_NOMEM;
    } else {
        for (int64_t k = J->tid; k < J->nrows; k += J->nthreads)
            one_row(J, J->rows[k], qd, s, vis, acc);
    }
    free(qd);
    free(acc);
    free(s);
    free(vis);
    return NULL;
}

/* ------------------------------------------------------------------ driver */

int mtv_oracle_run(int B, int N, int H, int max_kv, int64_t num_slots,
                   const uint16_t* q, const uint16_t* kv_pool,
                   const int32_t* page_table, const int32_t* seq_lens,
                   const uint32_t* tree_mask, double scale,
                   const int64_t* rows, int64_t nrows,
                   uint16_t* out_bf16, float* lse_f32,
                   double* out_f64, double* lse_f64, int threads)
{
    if (!q || !kv_pool || !page_table || !seq_lens || !tree_mask || !out_bf16 || !lse_f32)
        return MTV_ORACLE_ERR_ARG;
    if (B < 1 || N < 1 || H < 1 || max_kv < N || num_slots < 1)
        return MTV_ORACLE_ERR_ARG;
    if (threads < 1)
        threads = 1;
    const int W = (N + 31) / 32;
    const int64_t per_seq = (int64_t)N * H;
    const int64_t total = (int64_t)B * per_seq;
    if (rows) {
        for (int64_t k = 0; k < nrows; ++k)
            if (rows[k] < 0 || rows[k] >= total)
                return MTV_ORACLE_ERR_ARG;
    }

    int rc = MTV_ORACLE_OK;
    for (int b = 0; b < B && rc == MTV_ORACLE_OK; ++b) {
        const int S = seq_lens[b];
        if (S < N || S > max_kv)
            return MTV_ORACLE_ERR_SEQLEN;

        /* rows of this sequence that were asked for */
        int64_t cnt = 0;
        int64_t* mine = (int64_t*)malloc(sizeof(int64_t) * (size_t)per_seq);
        if (!mine)
            return MTV_ORACLE_ERR_NOMEM;
        if (rows) {
            for (int64_t k = 0; k < nrows; ++k)
                if (rows[k] / per_seq == b)
                    mine[cnt++] = rows[k];
        } else {
            for (int64_t r = 0; r < per_seq; ++r)
                mine[cnt++] = (int64_t)b * per_seq + r;
        }
        if (cnt == 0) {
            free(mine);
            continue;
        }

        /* gather: K[p] = pool[page_table[b][p]], widened to double */
        double* K = (double*)malloc(sizeof(double) * (size_t)S * D_QK);
        if (!K) {
            free(mine);
            return MTV_ORACLE_ERR_NOMEM;
        }
        for (int p = 0; p < S; ++p) {
            int32_t slot = page_table[(int64_t)b * max_kv + p];
            if (slot < 0 || (int64_t)slot >= num_slots) {
                free(K);
                free(mine);
                return MTV_ORACLE_ERR_INDEX;
            }
            const uint16_t* src = kv_pool + (int64_t)slot * D_QK;
            for (int d = 0; d < D_QK; ++d)
                K[(int64_t)p * D_QK + d] = mtv_oracle_bf16_to_f64(src[d]);
        }

        int nt = threads;
        if (nt > cnt)
            nt = (int)cnt;
        row_job* jobs = (row_job*)calloc((size_t)nt, sizeof(row_job));
        pthread_t* tids = (pthread_t*)calloc((size_t)nt, sizeof(pthread_t));
        if (!jobs || !tids) {
            free(jobs);
            free(tids);
            free(K);
            free(mine);
            return MTV_ORACLE_ERR_NOMEM;
        }
        for (int t = 0; t < nt; ++t) {
            row_job* J = &jobs[t];
            J->N = N;
            J->H = H;
            J->W = W;
            J->S = S;
            J->b = b;
            J->q = q;
            J->K = K;
            J->tree_mask = tree_mask;
            J->scale = scale;
            J->rows = mine;
            J->nrows = cnt;
            J->out_bf16 = out_bf16;
            J->lse_f32 = lse_f32;
            J->out_f64 = out_f64;
            J->lse_f64 = lse_f64;
            J->tid = t;
            J->nthreads = nt;
            J->err = 0;
        }
        int started = 0;
        for (int t = 1; t < nt; ++t) {
            if (pthread_create(&tids[t], NULL, row_worker, &jobs[t]) != 0)
                break;
            started = t;
        }
        /* any worker that could not be started is run on this thread */
        for (int t = started + 1; t < nt; ++t)
            row_worker(&jobs[t]);
        row_worker(&jobs[0]);
        for (int t = 1; t <= started; ++t)
            pthread_join(tids[t], NULL);
        for (int t = 0; t < nt; ++t)
            if (jobs[t].err)
                rc = jobs[t].err;
        free(jobs);
        free(tids);
        free(K);
        free(mine);
    }
    return rc;
}
