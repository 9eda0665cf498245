/*
 * oracle.c -- plain, slow CPU oracle for the lightning-indexer score + top-k,
 * and for the sparse attention that consumes the selected rows (second half
 * of this file).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library.  The GPU product
 * path never links, imports or calls it, and it shares no code, header,
 * table or helper with the GPU path.
 *
 * What it computes (one query token t at absolute position pos_t):
 *
 *   1. Visible rows.  A compressed KV row j summarises the r raw tokens
 *      r*j .. r*j+r-1 and becomes visible once the last of them has been
 *      seen, i.e. when r*j + r - 1 <= pos_t.  So the visible rows are
 *      j = 0 .. n_t-1 with n_t = floor((pos_t + 1) / r), clamped to [0, N].
 *      ("How I made DeepSeek 12x faster on a Mac Studio", section
 *      "1: the kernels": the lightning indexer scores *compressed* KV.)
 *
 *   2. Score of a visible row:
 *        s[t,j] = sum over index heads h of  w[t,h] * max(0, q[t,h,:] . k[j,:])
 *      where every index head of token t is dotted with the same compressed
 *      row k[j].
 *
 *   3. Selection: the min(n_t, topk) best rows under the order
 *      (score descending, row index ascending) -- i.e. among equal scores the
 *      lower row wins.  ("1: the kernels" on the same page: the indexer keeps
 *      the top 512 rows per token; the streaming top-k there is stated to
 *      give byte-identical output to a full sort, so the oracle *is* the
 *      full sort.)
 *
 *   4. Output: the selected rows in ascending row order, then -1 padding up
 *      to topk entries.  When every visible row fits (n_t <= topk) this is
 *      exactly 0 .. n_t-1 ("How I turned one oversized DeepSeek optimization
 *      into three merged oMLX PRs", section "3. Do not rank candidates when
 *      every candidate wins": the same sequential indices are produced).
 *      With n_t = 0 the row is all -1.
 *
 * Arithmetic: fp16 / bf16 inputs are decoded exactly to double (decoders
 * written from the IEEE 754 binary16 definition and from bfloat16 being the
 * top half of an IEEE binary32); every product, dot product, ReLU, weight
 * multiply and head sum is done in double; the sort compares doubles.
 * Non-finite inputs are rejected (status ORACLE_ERR_NONFINITE).
 *
 * Nothing here is blocked, fused or reordered: per token it scores every
 * visible row, sorts all of them, takes the first m, and sorts those by row.
 * Threads (pthreads) only split the token list; each token is computed by
 * one thread from start to finish.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F16 1
#define ORACLE_BF16 2

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_NONFINITE (-2)
#define ORACLE_ERR_NOMEM (-3)

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_half_to_double(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 10) & 0x1F;
    int frac = bits & 0x3FF;
    double mag;
    if (expo == 0x1F)
        mag = frac ? NAN : INFINITY;
    else if (expo == 0)
        mag = ldexp((double)frac, -24);              /* subnormal: frac * 2^-14 * 2^-10 */
    else
        mag = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/2^10) * 2^(expo-15) */
    return sign ? -mag : mag;
}

/* bfloat16: the upper 16 bits of an IEEE binary32 -- 1 sign bit, 8 exponent
 * bits (bias 127), 7 fraction bits. */
double oracle_bf16_to_double(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 7) & 0xFF;
    int frac = bits & 0x7F;
    double mag;
    if (expo == 0xFF)
        mag = frac ? NAN : INFINITY;
    else if (expo == 0)
        mag = ldexp((double)frac, -133);              /* frac * 2^-126 * 2^-7 */
    else
        mag = ldexp((double)(128 + frac), expo - 134); /* (1 + frac/2^7) * 2^(expo-127) */
    return sign ? -mag : mag;
}

static double decode(uint16_t bits, int dtype)
{
    return dtype == ORACLE_F16 ? oracle_half_to_double(bits) : oracle_bf16_to_double(bits);
}

/* Round a double to the nearest value with `sig` significant bits (ties to
 * even), for a format whose smallest normal exponent is emin and whose
 * subnormals share the quantum 2^(emin - sig + 1); returns the integer
 * significand n and the exponent E of the result n * 2^(E - sig + 1) (n <
 * 2^(sig-1) only for subnormals).  a > 0. */
static void round_sig(double a, int sig, int emin, double *n, int *E)
{
    int ex;
    frexp(a, &ex);        /* a = m * 2^ex, 0.5 <= m < 1: leading bit 2^(ex-1) */
    int e = ex - 1;
    if (e < emin)
        e = emin;         /* subnormal range: fixed quantum */
    double q = ldexp(1.0, e - sig + 1);
    double r = nearbyint(a / q); /* a / q is exact (power-of-two divisor); ties to even */
    if (r >= ldexp(1.0, sig)) { /* carried into the next binade */
        r = ldexp(1.0, sig - 1);
        ++e;
    }
    *n = r;
    *E = e;
}

/* double -> IEEE binary16 bits, round to nearest even; overflow -> infinity. */
uint16_t oracle_double_to_half(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v), n;
    int E;
    if (isnan(v))
        return 0x7E00;
    if (a == 0.0)
        return sign;
    round_sig(a, 11, -14, &n, &E);
    if (n < 1024.0) /* subnormal (or zero) */
        return (uint16_t)(sign | (uint16_t)n);
    if (E + 15 >= 31)
        return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | ((E + 15) << 10) | ((int)n - 1024));
}

/* double -> bfloat16 bits, round to nearest even; overflow -> infinity. */
uint16_t oracle_double_to_bf16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v), n;
    int E;
    if (isnan(v))
        return 0x7FC0;
    if (a == 0.0)
        return sign;
    round_sig(a, 8, -126, &n, &E);
    if (n < 128.0)
        return (uint16_t)(sign | (uint16_t)n);
    if (E + 127 >= 255)
        return (uint16_t)(sign | 0x7F80);
    return (uint16_t)(sign | ((E + 127) << 7) | ((int)n - 128));
}

/* Number of compressed rows visible to a token at absolute position pos:
 * row j is visible iff ratio*j + ratio - 1 <= pos and j < N. */
int64_t oracle_visible_rows(int64_t pos, int64_t ratio, int64_t n_rows)
{
    int64_t n;
    if (pos < 0)
        return 0;
    n = (pos + 1) / ratio;
    if (n > n_rows)
        n = n_rows;
    return n;
}

typedef struct {
    double score;
    int64_t row;
} scored_row;

/* Order of selection: higher score first; among equal scores, lower row first. */
static int by_score_desc_row_asc(const void *pa, const void *pb)
{
    const scored_row *a = (const scored_row *)pa;
    const scored_row *b = (const scored_row *)pb;
    if (a->score > b->score)
        return -1;
    if (a->score < b->score)
        return 1;
    if (a->row < b->row)
        return -1;
    if (a->row > b->row)
        return 1;
    return 0;
}

static int by_row_asc(const void *pa, const void *pb)
{
    int64_t a = *(const int64_t *)pa;
    int64_t b = *(const int64_t *)pb;
    return (a > b) - (a < b);
}

typedef struct {
    /* problem */
    const uint16_t *q;   /* [T][H][D] raw fp16/bf16 bits */
    const double *k;     /* [N][D] decoded rows */
    const float *w;      /* [T][H] */
    const int32_t *pos;  /* [T] */
    int64_t T, N;
    int H, D, dtype, ratio, topk;
    const int64_t *tokens; /* which tokens to compute (length n_out) */
    int64_t n_out;
    int32_t *out;        /* [n_out][topk] */
    double *scores;      /* optional [n_out][N]; -inf where not visible */
    /* threading */
    int nthreads;
    int tid;
    int status;
} job;

static void *run_job(void *arg)
{
    job *jb = (job *)arg;
    const int H = jb->H, D = jb->D;
    double *qt = (double *)malloc(sizeof(double) * (size_t)H * (size_t)D);
    scored_row *rows = (scored_row *)malloc(sizeof(scored_row) * (size_t)(jb->N > 0 ? jb->N : 1));
    int64_t *chosen = (int64_t *)malloc(sizeof(int64_t) * (size_t)(jb->topk > 0 ? jb->topk : 1));
    int64_t i;
    jb->status = ORACLE_OK;
    if (!qt || !rows || !chosen) {
        jb->status = ORACLE_ERR_NOMEM;
        goto done;
    }
    for (i = jb->tid; i < jb->n_out; i += jb->nthreads) {
        const int64_t t = jb->tokens ? jb->tokens[i] : i;
        const float *wt = jb->w + t * H;
        int32_t *o = jb->out + i * jb->topk;
        const int64_t n = oracle_visible_rows(jb->pos[t], jb->ratio, jb->N);
        int64_t j, m, c;
        int h, d;
        for (h = 0; h < H; ++h) {
            if (!isfinite((double)wt[h])) {
                jb->status = ORACLE_ERR_NONFINITE;
                goto done;
            }
            for (d = 0; d < D; ++d) {
                double v = decode(jb->q[(t * H + h) * D + d], jb->dtype);
                if (!isfinite(v)) {
                    jb->status = ORACLE_ERR_NONFINITE;
                    goto done;
                }
                qt[h * D + d] = v;
            }
        }
        /* score every visible row */
        for (j = 0; j < n; ++j) {
            const double *kj = jb->k + j * D;
            double s = 0.0;
            for (h = 0; h < H; ++h) {
                double x = 0.0;
                for (d = 0; d < D; ++d)
                    x += qt[h * D + d] * kj[d];
                s += (double)wt[h] * (x > 0.0 ? x : 0.0);
            }
            rows[j].score = s;
            rows[j].row = j;
        }
        if (jb->scores) {
            double *so = jb->scores + i * jb->N;
            for (j = 0; j < jb->N; ++j)
                so[j] = j < n ? rows[j].score : -INFINITY;
        }
        /* full sort, keep the first m, emit them in ascending row order */
        qsort(rows, (size_t)n, sizeof(scored_row), by_score_desc_row_asc);
        m = n < jb->topk ? n : jb->topk;
        for (c = 0; c < m; ++c)
            chosen[c] = rows[c].row;
        qsort(chosen, (size_t)m, sizeof(int64_t), by_row_asc);
        for (c = 0; c < jb->topk; ++c)
            o[c] = c < m ? (int32_t)chosen[c] : -1;
    }
done:
    free(qt);
    free(rows);
    free(chosen);
    return NULL;
}

/*
 * Score and select for the tokens listed in `tokens` (or all T tokens when
 * `tokens` is NULL, in which case n_out must equal T).
 *
 *   q      [T][H][D]  raw fp16 (dtype 1) or bf16 (dtype 2) bits
 *   k      [N][D]     raw bits, same dtype
 *   w      [T][H]     float32 head weights
 *   pos    [T]        int32 absolute positions
 *   out    [n_out][topk] int32: ascending selected rows, then -1
 *   scores optional [n_out][N] double: the score of every visible row,
 *          -inf for rows the token cannot see
 *   threads  worker threads (<= 0: 1)
 *
 * Returns ORACLE_OK, ORACLE_ERR_ARG, ORACLE_ERR_NONFINITE or ORACLE_ERR_NOMEM.
 */
int oracle_score_topk(const uint16_t *q, const uint16_t *k, const float *w, const int32_t *pos,
                      int64_t T, int64_t N, int H, int D, int dtype, int ratio, int topk,
                      const int64_t *tokens, int64_t n_out, int32_t *out, double *scores,
                      int threads)
{
    double *kd;
    job *jobs;
    pthread_t *tids;
    int *started;
    int64_t i, need_rows = 0;
    int th, status = ORACLE_OK;

    if (T < 0 || N < 0 || H < 1 || D < 1 || ratio < 1 || topk < 1 || n_out < 0)
        return ORACLE_ERR_ARG;
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16)
        return ORACLE_ERR_ARG;
    if (!tokens && n_out != T)
        return ORACLE_ERR_ARG;
    if (n_out > 0 && (!q || !w || !pos || !out))
        return ORACLE_ERR_ARG;
    if (N > 0 && n_out > 0 && !k)
        return ORACLE_ERR_ARG;
    for (i = 0; i < n_out; ++i) {
        int64_t t = tokens ? tokens[i] : i;
        int64_t n;
        if (t < 0 || t >= T)
            return ORACLE_ERR_ARG;
        n = oracle_visible_rows(pos[t], ratio, N);
        if (n > need_rows)
            need_rows = n;
    }
    if (threads < 1)
        threads = 1;

    /* decode only the rows some requested token can see */
    kd = (double *)malloc(sizeof(double) * (size_t)(need_rows > 0 ? need_rows * D : 1));
    if (!kd)
        return ORACLE_ERR_NOMEM;
    for (i = 0; i < need_rows * D; ++i) {
        kd[i] = decode(k[i], dtype);
        if (!isfinite(kd[i])) {
            free(kd);
            return ORACLE_ERR_NONFINITE;
        }
    }

    jobs = (job *)calloc((size_t)threads, sizeof(job));
    tids = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    started = (int *)calloc((size_t)threads, sizeof(int));
    if (!jobs || !tids || !started) {
        free(kd);
        free(jobs);
        free(tids);
        free(started);
        return ORACLE_ERR_NOMEM;
    }
    for (th = 0; th < threads; ++th) {
        job *jb = &jobs[th];
        jb->q = q;
        jb->k = kd;
        jb->w = w;
        jb->pos = pos;
        jb->T = T;
        jb->N = N;
        jb->H = H;
        jb->D = D;
        jb->dtype = dtype;
        jb->ratio = ratio;
        jb->topk = topk;
        jb->tokens = tokens;
        jb->n_out = n_out;
        jb->out = out;
        jb->scores = scores;
        jb->nthreads = threads;
        jb->tid = th;
    }
    /* thread 0's share runs on the calling thread; a share whose thread
     * cannot be started also runs here, so every token is always computed */
    for (th = 1; th < threads; ++th)
        started[th] = pthread_create(&tids[th], NULL, run_job, &jobs[th]) == 0;
    run_job(&jobs[0]);
    for (th = 1; th < threads; ++th) {
        if (started[th])
            pthread_join(tids[th], NULL);
        else
            run_job(&jobs[th]);
    }
    for (th = 0; th < threads; ++th)
        if (jobs[th].status != ORACLE_OK)
            status = jobs[th].status;
    free(kd);
    free(jobs);
    free(tids);
    free(started);
    return status;
}


/* ======================================================================== *
 * Sparse attention over the selected rows (the consumer of the indices).
 *
 * The pages describe the consumer as compressed attention that concatenates
 * local key/value state with pooled (compressed) key/value state and runs
 * ordinary dense attention over the result; the native kernel takes the
 * pooled indices ("How I turned one oversized DeepSeek optimization into
 * three merged oMLX PRs", section "1. Route ratio-128 prefill through native
 * attention"), and the pooled rows a token uses are the ones its indexer
 * selected ("How I made DeepSeek 12x faster on a Mac Studio", opening of
 * section "1: the kernels").
 *
 * For token t at absolute position pos_t and attention head h:
 *
 *   rows R(t) = local rows p = max(0, pos_t - window + 1) .. min(pos_t, L-1)
 *               of the raw cache (none when pos_t < 0 or window == 0),
 *             + pooled rows j = idx[t][i] for every entry i with idx >= 0
 *               (entries < 0 are padding; an entry >= N is an error),
 *               or, in the all-visible form (oracle_sparse_attention_all),
 *               every pooled row the token can see: j = 0 .. n_t - 1 with
 *               n_t = oracle_visible_rows(pos_t, ratio, N) -- the
 *               sequential pooled indices that ratio-128 layers attend to
 *               without an indexer (same section of the oMLX page)
 *   s_r       = scale * sum_d q[t,h,d] * key_r[d]
 *   o[t,h,:]  = sum_r  exp(s_r - max_r s) / sum_r' exp(s_r' - max s) * value_r
 *             = 0 when R(t) is empty.
 *
 * Keys and values are shared by all heads.  Everything is decoded exactly
 * to double and computed in double; nothing is blocked or reordered: per
 * (token, head) it scores every row of R(t), takes the largest score, forms
 * the weights and sums.
 * ======================================================================== */

typedef struct {
    const uint16_t *q;        /* [T][HA][DK] */
    const double *kp, *vp;    /* [N][DK], [N][DV] decoded */
    const double *kl, *vl;    /* [L][DK], [L][DV] decoded */
    const int32_t *idx, *pos; /* [T][topk], [T] */
    int64_t T, N, L;
    int HA, DK, DV, topk, window, dtype;
    int ratio;                /* > 0: every visible pooled row, idx unused */
    double scale;
    const int64_t *tokens;
    int64_t n_out;
    double *out;              /* [n_out][HA][DV] */
    int nthreads, tid, status;
} attn_job;

static void *run_attn_job(void *arg)
{
    attn_job *jb = (attn_job *)arg;
    const int HA = jb->HA, DK = jb->DK, DV = jb->DV;
    const int64_t cap = (jb->ratio > 0 ? jb->N : (int64_t)jb->topk) + (jb->window > 0 ? jb->window : 0);
    const double **krow = (const double **)malloc(sizeof(double *) * (size_t)(cap > 0 ? cap : 1));
    const double **vrow = (const double **)malloc(sizeof(double *) * (size_t)(cap > 0 ? cap : 1));
    double *s = (double *)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1));
    double *qh = (double *)malloc(sizeof(double) * (size_t)DK);
    int64_t i;
    jb->status = ORACLE_OK;
    if (!krow || !vrow || !s || !qh) {
        jb->status = ORACLE_ERR_NOMEM;
        goto done;
    }
    for (i = jb->tid; i < jb->n_out; i += jb->nthreads) {
        const int64_t t = jb->tokens ? jb->tokens[i] : i;
        const int64_t p = jb->pos[t];
        int64_t nr = 0, r, lo, hi;
        int h, d, e;
        /* the row set R(t): local rows first, then the listed pooled rows */
        if (p >= 0 && jb->window > 0) {
            lo = p - jb->window + 1;
            if (lo < 0)
                lo = 0;
            hi = p < jb->L - 1 ? p : jb->L - 1;
            for (r = lo; r <= hi; ++r) {
                krow[nr] = jb->kl + r * DK;
                vrow[nr] = jb->vl + r * DV;
                ++nr;
            }
        }
        if (jb->ratio > 0) {
            const int64_t nv = oracle_visible_rows(p, jb->ratio, jb->N);
            for (r = 0; r < nv; ++r) {
                krow[nr] = jb->kp + r * DK;
                vrow[nr] = jb->vp + r * DV;
                ++nr;
            }
        }
        for (e = 0; e < jb->topk; ++e) {
            const int32_t j = jb->idx[t * jb->topk + e];
            if (j < 0)
                continue;
            if (j >= jb->N) {
                jb->status = ORACLE_ERR_ARG;
                goto done;
            }
            krow[nr] = jb->kp + (int64_t)j * DK;
            vrow[nr] = jb->vp + (int64_t)j * DV;
            ++nr;
        }
        for (h = 0; h < HA; ++h) {
            double *o = jb->out + (i * HA + h) * DV;
            double m = -INFINITY, z = 0.0;
            for (d = 0; d < DK; ++d) {
                qh[d] = decode(jb->q[(t * HA + h) * DK + d], jb->dtype);
                if (!isfinite(qh[d])) {
                    jb->status = ORACLE_ERR_NONFINITE;
                    goto done;
                }
            }
            for (d = 0; d < DV; ++d)
                o[d] = 0.0;
            if (nr == 0)
                continue;
            for (r = 0; r < nr; ++r) {
                double x = 0.0;
                for (d = 0; d < DK; ++d)
                    x += qh[d] * krow[r][d];
                s[r] = jb->scale * x;
                if (s[r] > m)
                    m = s[r];
            }
            for (r = 0; r < nr; ++r) {
                s[r] = exp(s[r] - m);
                z += s[r];
            }
            for (r = 0; r < nr; ++r) {
                const double a = s[r] / z;
                for (d = 0; d < DV; ++d)
                    o[d] += a * vrow[r][d];
            }
        }
    }
done:
    free(krow);
    free(vrow);
    free(s);
    free(qh);
    return NULL;
}

static double *decode_all(const uint16_t *bits, int64_t n, int dtype, int *status)
{
    int64_t i;
    double *x = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    if (!x) {
        *status = ORACLE_ERR_NOMEM;
        return NULL;
    }
    for (i = 0; i < n; ++i) {
        x[i] = decode(bits[i], dtype);
        if (!isfinite(x[i])) {
            *status = ORACLE_ERR_NONFINITE;
            free(x);
            return NULL;
        }
    }
    return x;
}

/*
 * Sparse attention for the tokens listed in `tokens` (or all T when NULL, in
 * which case n_out must equal T).
 *
 *   q    [T][HA][DK]  raw fp16 (dtype 1) or bf16 (dtype 2) bits
 *   kp   [N][DK], vp [N][DV]   pooled key / value rows, same dtype
 *   kl   [L][DK], vl [L][DV]   raw (local) key / value rows by absolute position
 *   idx  [T][topk] int32: pooled rows of each token, -1 = padding
 *   pos  [T] int32 absolute positions
 *   out  [n_out][HA][DV] double
 *   ratio > 0 selects the all-visible form (idx unused, topk 0)
 *
 * Returns ORACLE_OK, ORACLE_ERR_ARG, ORACLE_ERR_NONFINITE or ORACLE_ERR_NOMEM.
 */
static int attention_common(const uint16_t *q, const uint16_t *kp, const uint16_t *vp,
                            const uint16_t *kl, const uint16_t *vl, const int32_t *idx,
                            const int32_t *pos, int64_t T, int64_t N, int64_t L, int HA, int DK,
                            int DV, int topk, int ratio, int window, double scale, int dtype,
                            const int64_t *tokens, int64_t n_out, double *out, int threads)
{
    double *kpd = NULL, *vpd = NULL, *kld = NULL, *vld = NULL;
    attn_job *jobs = NULL;
    pthread_t *tids = NULL;
    int *started = NULL;
    int64_t i;
    int th, status = ORACLE_OK;

    if (T < 0 || N < 0 || L < 0 || HA < 1 || DK < 1 || DV < 1 || topk < 0 || window < 0 ||
        n_out < 0 || !isfinite(scale))
        return ORACLE_ERR_ARG;
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16)
        return ORACLE_ERR_ARG;
    if (!tokens && n_out != T)
        return ORACLE_ERR_ARG;
    if (n_out > 0 && (!q || !pos || !out || (topk > 0 && !idx)))
        return ORACLE_ERR_ARG;
    if ((N > 0 && (!kp || !vp)) || (L > 0 && (!kl || !vl)))
        return ORACLE_ERR_ARG;
    for (i = 0; i < n_out; ++i)
        if (tokens && (tokens[i] < 0 || tokens[i] >= T))
            return ORACLE_ERR_ARG;
    if (threads < 1)
        threads = 1;
    kpd = decode_all(kp, N * DK, dtype, &status);
    if (kpd)
        vpd = decode_all(vp, N * DV, dtype, &status);
    if (vpd)
        kld = decode_all(kl, L * DK, dtype, &status);
    if (kld)
        vld = decode_all(vl, L * DV, dtype, &status);
    if (!vld)
        goto out;
    jobs = (attn_job *)calloc((size_t)threads, sizeof(attn_job));
    tids = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    started = (int *)calloc((size_t)threads, sizeof(int));
    if (!jobs || !tids || !started) {
        status = ORACLE_ERR_NOMEM;
        goto out;
    }
    for (th = 0; th < threads; ++th) {
        attn_job *jb = &jobs[th];
        jb->q = q;
        jb->kp = kpd;
        jb->vp = vpd;
        jb->kl = kld;
        jb->vl = vld;
        jb->idx = idx;
        jb->pos = pos;
        jb->T = T;
        jb->N = N;
        jb->L = L;
        jb->HA = HA;
        jb->DK = DK;
        jb->DV = DV;
        jb->topk = topk;
        jb->ratio = ratio;
        jb->window = window;
        jb->dtype = dtype;
        jb->scale = scale;
        jb->tokens = tokens;
        jb->n_out = n_out;
        jb->out = out;
        jb->nthreads = threads;
        jb->tid = th;
    }
    for (th = 1; th < threads; ++th)
        started[th] = pthread_create(&tids[th], NULL, run_attn_job, &jobs[th]) == 0;
    run_attn_job(&jobs[0]);
    for (th = 1; th < threads; ++th) {
        if (started[th])
            pthread_join(tids[th], NULL);
        else
            run_attn_job(&jobs[th]);
    }
    for (th = 0; th < threads; ++th)
        if (jobs[th].status != ORACLE_OK)
            status = jobs[th].status;
out:
    free(kpd);
    free(vpd);
    free(kld);
    free(vld);
    free(jobs);
    free(tids);
    free(started);
    return status;
}

int oracle_sparse_attention(const uint16_t *q, const uint16_t *kp, const uint16_t *vp,
                            const uint16_t *kl, const uint16_t *vl, const int32_t *idx,
                            const int32_t *pos, int64_t T, int64_t N, int64_t L, int HA, int DK,
                            int DV, int topk, int window, double scale, int dtype,
                            const int64_t *tokens, int64_t n_out, double *out, int threads)
{
    return attention_common(q, kp, vp, kl, vl, idx, pos, T, N, L, HA, DK, DV, topk, 0, window,
                            scale, dtype, tokens, n_out, out, threads);
}

/*
 * The all-visible form: every token attends to its local rows plus every
 * pooled row it can see (rows 0 .. n_t - 1, n_t = oracle_visible_rows(pos_t,
 * ratio, N)); no index list.  ratio >= 1.  Same arguments otherwise.
 */
int oracle_sparse_attention_all(const uint16_t *q, const uint16_t *kp, const uint16_t *vp,
                                const uint16_t *kl, const uint16_t *vl, const int32_t *pos,
                                int64_t T, int64_t N, int64_t L, int HA, int DK, int DV, int ratio,
                                int window, double scale, int dtype, const int64_t *tokens,
                                int64_t n_out, double *out, int threads)
{
    if (ratio < 1)
        return ORACLE_ERR_ARG;
    return attention_common(q, kp, vp, kl, vl, NULL, pos, T, N, L, HA, DK, DV, 0, ratio, window,
                            scale, dtype, tokens, n_out, out, threads);
}

/* ======================================================================== *
 * The indexer's query projection, the step just before the scorer: the
 * query rows of the index heads are a linear map of each token's query
 * input ("How I made DeepSeek 12x faster on a Mac Studio" names the big Q
 * projection ahead of the indexer; its weights are model parameters, here
 * synthetic).  For token t and output feature o = h * D + d:
 *
 *   q[t][o] = round_dtype( sum_i x[t][i] * wq[o][i] )
 *
 * x [T][d_in] and wq [O][d_in] are raw fp16/bf16 bits; the sum is taken in
 * double over exactly decoded operands and rounded once, to nearest even,
 * into the storage type (the scorer reads q in that type).  Non-finite
 * inputs or results are rejected.
 * ======================================================================== */

typedef struct {
    const uint16_t *x, *wq;
    int64_t T, din, O;
    int dtype;
    uint16_t *q;
    int nthreads, tid, status;
} proj_job;

static void *run_proj_job(void *arg)
{
    proj_job *jb = (proj_job *)arg;
    int64_t t, o, i;
    jb->status = ORACLE_OK;
    for (t = jb->tid; t < jb->T; t += jb->nthreads) {
        for (o = 0; o < jb->O; ++o) {
            double acc = 0.0;
            for (i = 0; i < jb->din; ++i) {
                const double a = decode(jb->x[t * jb->din + i], jb->dtype);
                const double b = decode(jb->wq[o * jb->din + i], jb->dtype);
                if (!isfinite(a) || !isfinite(b)) {
                    jb->status = ORACLE_ERR_NONFINITE;
                    return NULL;
                }
                acc += a * b;
            }
            jb->q[t * jb->O + o] = jb->dtype == ORACLE_F16 ? oracle_double_to_half(acc)
                                                          : oracle_double_to_bf16(acc);
            if (!isfinite(decode(jb->q[t * jb->O + o], jb->dtype))) {
                jb->status = ORACLE_ERR_NONFINITE;
                return NULL;
            }
        }
    }
    return NULL;
}

int oracle_project_q(const uint16_t *x, const uint16_t *wq, int64_t T, int64_t din, int64_t O,
                     int dtype, uint16_t *q, int threads)
{
    proj_job *jobs;
    pthread_t *tids;
    int *started;
    int th, status = ORACLE_OK;
    if (T < 0 || din < 1 || O < 1 || (dtype != ORACLE_F16 && dtype != ORACLE_BF16))
        return ORACLE_ERR_ARG;
    if (T > 0 && (!x || !wq || !q))
        return ORACLE_ERR_ARG;
    if (threads < 1)
        threads = 1;
    jobs = (proj_job *)calloc((size_t)threads, sizeof(proj_job));
    tids = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    started = (int *)calloc((size_t)threads, sizeof(int));
    if (!jobs || !tids || !started) {
        free(jobs);
        free(tids);
        free(started);
        return ORACLE_ERR_NOMEM;
    }
    for (th = 0; th < threads; ++th) {
        jobs[th].x = x;
        jobs[th].wq = wq;
        jobs[th].T = T;
        jobs[th].din = din;
        jobs[th].O = O;
        jobs[th].dtype = dtype;
        jobs[th].q = q;
        jobs[th].nthreads = threads;
        jobs[th].tid = th;
    }
    for (th = 1; th < threads; ++th)
        started[th] = pthread_create(&tids[th], NULL, run_proj_job, &jobs[th]) == 0;
    run_proj_job(&jobs[0]);
    for (th = 1; th < threads; ++th) {
        if (started[th])
            pthread_join(tids[th], NULL);
        else
            run_proj_job(&jobs[th]);
    }
    for (th = 0; th < threads; ++th)
        if (jobs[th].status != ORACLE_OK)
            status = jobs[th].status;
    free(jobs);
    free(tids);
    free(started);
    return status;
}
