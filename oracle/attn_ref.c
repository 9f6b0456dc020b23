/*
 * attn_ref.c — CPU fp64 oracle for exact attention forward.
 *
 * TEST INFRASTRUCTURE: a plain, slow, obviously correct implementation of
 * the attention definition. Only the test suite, the smoke check and the
 * bench's CPU-baseline leg load it. It shares no code with the GPU library.
 *
 * What it computes is the plain definition, written out step by step:
 *   [naive-attn] cishoon.github.io "flashattention" post, section 1.1.2:
 *     Attention(Q,K,V) = softmax(Q K^T / sqrt(d)) V, the softmax taken per
 *     row over the key axis, made safe by subtracting the row maximum
 *     (item 3), and o_i = sum_j alpha_ij v_j (item 4). Section 2 spells out
 *     the same three steps as separate materialised passes (scores, softmax,
 *     P.V); this file keeps that order for one query row at a time.
 *   [v2-naive] "Flash Attention（二）v2版本朴素实现 cuda core", section 3.3:
 *     the scale is multiplied into the score; section 3.4: query row i sees
 *     key j only when j <= i under the causal mask (diagonal included).
 *   [FA2-principles] "Flash Attention v2 的核心优化原理与工程实现", section 4:
 *     the row statistics (max and sum) are written next to O; they are
 *     returned here folded into one log-sum-exp, lse_i = m_i + ln(l_i).
 *
 * The scale is the caller's fp32 value widened to double, so that the oracle
 * and any other implementation use the identical number.
 *
 * Grouped-query attention ([FA2-principles], References item 5: Flash
 * Attention combined with GQA, K/V shared by groups of query heads): with
 * H_kv K/V heads, query head h reads K/V head h / (H / H_kv), i.e. groups of
 * H / H_kv consecutive query heads share one K/V head. H_kv = H is ordinary
 * multi-head attention, H_kv = 1 multi-query attention.
 *
 * Pinned by tests/test_oracle_pins.py against closed forms, invariants the
 * pages state (rows of P sum to 1, constant V, Q = 0 mean, unit-basis probe,
 * causal row 0, N = 1 and N = 2 closed forms), brute force on tiny inputs
 * against a library softmax, and the pages' printed worked values.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#include "../include/attn_ref.h"

/* ---- exact decoding of the input formats ------------------------------ */

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 mantissa bits. */
static double decode_f16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* zero / subnormal */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);     /* (1.m) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
static double decode_bf16(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static double decode_one(const void* base, int64_t idx, int dtype)
{
    if (dtype == ATTN_REF_F32) {
        float f;
        memcpy(&f, (const char*)base + idx * 4, 4);
        return (double)f;
    }
    uint16_t h;
    memcpy(&h, (const char*)base + idx * 2, 2);
    return dtype == ATTN_REF_F16 ? decode_f16(h) : decode_bf16(h);
}

int attn_ref_decode(const void* src, double* dst, int64_t n, int dtype)
{
    if (!src || !dst || n < 0)
        return ATTN_REF_EINVAL;
    if (dtype != ATTN_REF_F32 && dtype != ATTN_REF_F16 && dtype != ATTN_REF_BF16)
        return ATTN_REF_EINVAL;
    for (int64_t i = 0; i < n; i++)
        dst[i] = decode_one(src, i, dtype);
    return ATTN_REF_OK;
}

/* ---- one query row, straight from the definition ----------------------- */

typedef struct {
    const void *q, *k, *v;
    int64_t B, H, H_kv, N, d;
    int causal;
    double scale;
    int dtype;
    const int64_t* rows;   /* flat row ids */
    int64_t n_rows;
    double* o;             /* [n_rows, d] */
    double* lse;           /* [n_rows] or NULL */
    int64_t next;          /* shared work counter */
    int failed;
} job_t;

/* Computes output row `t` of the job: query row r = rows[t].
 * s_row has room for N doubles, qrow for d doubles. */
static void one_row(job_t* jb, int64_t t, double* s_row, double* qrow)
{
    const int64_t N = jb->N, d = jb->d;
    const int64_t r = jb->rows[t];
    const int64_t bh = r / N;          /* (b*H + h) */
    const int64_t i = r % N;           /* query position */
    const int64_t slice = bh * N * d;  /* element offset of the (b,h) slice of q */
    /* K/V head of query head h: h / (H / H_kv) */
    const int64_t b = bh / jb->H, h = bh % jb->H;
    const int64_t kv_slice = (b * jb->H_kv + h / (jb->H / jb->H_kv)) * N * d;

    /* visible keys: j in [0, n_vis) */
    const int64_t n_vis = jb->causal ? i + 1 : N;

    for (int64_t c = 0; c < d; c++)
        qrow[c] = decode_one(jb->q, slice + i * d + c, jb->dtype);

    /* step 1: scores s_ij = scale * (q_i . k_j), one materialised row of S */
    for (int64_t j = 0; j < n_vis; j++) {
        double dot = 0.0;
        for (int64_t c = 0; c < d; c++)
            dot += qrow[c] * decode_one(jb->k, kv_slice + j * d + c, jb->dtype);
        s_row[j] = jb->scale * dot;
    }

    /* step 2: safe softmax over the row */
    double m = -INFINITY;
    for (int64_t j = 0; j < n_vis; j++)
        if (s_row[j] > m)
            m = s_row[j];
    double l = 0.0;
    for (int64_t j = 0; j < n_vis; j++) {
        s_row[j] = exp(s_row[j] - m);   /* e_ij, overwrites s_ij */
        l += s_row[j];
    }
    for (int64_t j = 0; j < n_vis; j++)
        s_row[j] = s_row[j] / l;        /* p_ij */

    /* step 3: o_i = sum_j p_ij v_j */
    double* o = jb->o + t * d;
    for (int64_t c = 0; c < d; c++)
        o[c] = 0.0;
    for (int64_t j = 0; j < n_vis; j++) {
        const double p = s_row[j];
        for (int64_t c = 0; c < d; c++)
            o[c] += p * decode_one(jb->v, kv_slice + j * d + c, jb->dtype);
    }

    if (jb->lse)
        jb->lse[t] = m + log(l);
}

static void* worker(void* arg)
{
    job_t* jb = (job_t*)arg;
    double* s_row = (double*)malloc((size_t)jb->N * sizeof(double));
    double* qrow = (double*)malloc((size_t)jb->d * sizeof(double));
    if (!s_row || !qrow) {
        __atomic_store_n(&jb->failed, 1, __ATOMIC_SEQ_CST);
        free(s_row);
        free(qrow);
        return NULL;
    }
    for (;;) {
        int64_t t = __atomic_fetch_add(&jb->next, 1, __ATOMIC_RELAXED);
        if (t >= jb->n_rows)
            break;
        one_row(jb, t, s_row, qrow);
    }
    free(s_row);
    free(qrow);
    return NULL;
}

static int check_args(const void* q, const void* k, const void* v,
                      int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d,
                      int causal, float scale, int dtype)
{
    if (!q || !k || !v)
        return ATTN_REF_EINVAL;
    if (B <= 0 || H <= 0 || N <= 0 || d <= 0)
        return ATTN_REF_EINVAL;
    if (H_kv <= 0 || H % H_kv != 0)
        return ATTN_REF_EINVAL;
    if (causal != 0 && causal != 1)
        return ATTN_REF_EINVAL;
    if (!isfinite(scale))
        return ATTN_REF_EINVAL;
    if (dtype != ATTN_REF_F32 && dtype != ATTN_REF_F16 && dtype != ATTN_REF_BF16)
        return ATTN_REF_EINVAL;
    /* B*H*N*d must be addressable */
    if (B > INT64_MAX / H || B * H > INT64_MAX / N || B * H * N > INT64_MAX / d / 4)
        return ATTN_REF_EINVAL;
    return ATTN_REF_OK;
}

static int run_job(job_t* jb, int num_threads)
{
    if (num_threads <= 0) {
        long n = sysconf(_SC_NPROCESSORS_ONLN);
        num_threads = n > 0 ? (int)n : 1;
    }
    if (num_threads > jb->n_rows)
        num_threads = (int)(jb->n_rows > 0 ? jb->n_rows : 1);

    pthread_t* th = (pthread_t*)malloc((size_t)num_threads * sizeof(pthread_t));
    if (!th)
        return ATTN_REF_ENOMEM;
    int started = 0;
    for (int t = 0; t < num_threads; t++) {
        if (pthread_create(&th[t], NULL, worker, jb) != 0)
            break;
        started++;
    }
    if (started == 0)
        worker(jb);   /* no thread could start: do the work here */
    for (int t = 0; t < started; t++)
        pthread_join(th[t], NULL);
    free(th);
    return jb->failed ? ATTN_REF_ENOMEM : ATTN_REF_OK;
}

int attn_fwd_ref_rows_gqa(const void* q, const void* k, const void* v,
                          int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d,
                          int causal, float scale, int dtype,
                          const int64_t* rows, int64_t n_rows,
                          double* o_rows, double* lse_rows, int num_threads)
{
    int rc = check_args(q, k, v, B, H, H_kv, N, d, causal, scale, dtype);
    if (rc != ATTN_REF_OK)
        return rc;
    if (n_rows < 0 || (n_rows > 0 && (!rows || !o_rows)))
        return ATTN_REF_EINVAL;
    for (int64_t t = 0; t < n_rows; t++)
        if (rows[t] < 0 || rows[t] >= B * H * N)
            return ATTN_REF_EINVAL;
    if (n_rows == 0)
        return ATTN_REF_OK;

    job_t jb;
    memset(&jb, 0, sizeof jb);
    jb.q = q; jb.k = k; jb.v = v;
    jb.B = B; jb.H = H; jb.H_kv = H_kv; jb.N = N; jb.d = d;
    jb.causal = causal;
    jb.scale = (double)scale;
    jb.dtype = dtype;
    jb.rows = rows;
    jb.n_rows = n_rows;
    jb.o = o_rows;
    jb.lse = lse_rows;
    return run_job(&jb, num_threads);
}

int attn_fwd_ref_gqa(const void* q, const void* k, const void* v,
                     double* o_ref, double* lse_ref,
                     int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d,
                     int causal, float scale, int dtype, int num_threads)
{
    int rc = check_args(q, k, v, B, H, H_kv, N, d, causal, scale, dtype);
    if (rc != ATTN_REF_OK)
        return rc;
    if (!o_ref)
        return ATTN_REF_EINVAL;
    const int64_t n = B * H * N;
    int64_t* rows = (int64_t*)malloc((size_t)n * sizeof(int64_t));
    if (!rows)
        return ATTN_REF_ENOMEM;
    for (int64_t r = 0; r < n; r++)
        rows[r] = r;   /* every row, in storage order: o_rows == o_ref */
    rc = attn_fwd_ref_rows_gqa(q, k, v, B, H, H_kv, N, d, causal, scale, dtype,
                               rows, n, o_ref, lse_ref, num_threads);
    free(rows);
    return rc;
}

int attn_fwd_ref_rows(const void* q, const void* k, const void* v,
                      int64_t B, int64_t H, int64_t N, int64_t d,
                      int causal, float scale, int dtype,
                      const int64_t* rows, int64_t n_rows,
                      double* o_rows, double* lse_rows, int num_threads)
{
    return attn_fwd_ref_rows_gqa(q, k, v, B, H, H, N, d, causal, scale, dtype,
                                 rows, n_rows, o_rows, lse_rows, num_threads);
}

int attn_fwd_ref(const void* q, const void* k, const void* v,
                 double* o_ref, double* lse_ref,
                 int64_t B, int64_t H, int64_t N, int64_t d,
                 int causal, float scale, int dtype, int num_threads)
{
    return attn_fwd_ref_gqa(q, k, v, o_ref, lse_ref, B, H, H, N, d, causal, scale,
                            dtype, num_threads);
}

/* ---- backward: the chain rule of the definition above -------------------
 *
 * For one query row i (of query head h, K/V head h / (H/H_kv)), with the
 * visible keys J_i and the softmax row p_ij of the forward definition:
 *   o_i    = sum_j p_ij v_j
 *   D_i    = sum_c dO_ic o_ic
 *   dp_ij  = dO_i . v_j
 *   ds_ij  = p_ij (dp_ij - D_i)          (derivative through the softmax)
 *   dq_i   = scale sum_j ds_ij k_j        (s_ij = scale q_i . k_j)
 *   dk_j  += scale ds_ij q_i
 *   dv_j  += p_ij dO_i                    (o_i = sum_j p_ij v_j)
 * Every query row of every query head that shares a K/V head adds into that
 * head's dk and dv.
 *
 * Optional error scales: first-order magnitudes of the terms that a
 * computation rounding p, ds and o to a floating-point type perturbs. With
 * A_i = sum_c |dO_ic o_ic| and w_ij = |ds_ij| + p_ij A_i (relative rounding),
 *   eq_ic = scale sum_j w_ij |k_jc|,  ek_jc = scale sum_i w_ij |q_ic|,
 *   ev_jc = sum_i p_ij |dO_ic|;
 * with g_i = sum_c |dO_ic| and z_ij = 1 + p_ij g_i (absolute rounding, a
 * type's subnormal spacing),
 *   zq_ic = scale sum_j z_ij |k_jc|,  zk_jc = scale sum_i z_ij |q_ic|,
 *   zv_jc = sum_i |dO_ic|.
 */

typedef struct {
    const void *q, *dout;
    const double *kd, *vd;      /* this K/V slice, decoded, [N, d] */
    const double *ka;           /* |kd| */
    int64_t N, d;
    int causal;
    double scale;
    int dtype;
    int64_t q_head0;            /* b*H + h of the slice's first query head */
    int64_t row_begin, row_end; /* t in [0, G*N): head q_head0 + t/N, row t%N */
    double *dq, *eq;            /* [B,H,N,d] outputs (eq may be NULL) */
    double *zq;                 /* may be NULL */
    double *dk, *dv, *ek, *ev;  /* this worker's partial sums, [N, d] */
    double *zk, *zv;
    double *work;               /* 3N + 5d doubles */
} bwd_part_t;

static void bwd_row(bwd_part_t* w, int64_t t)
{
    const int64_t N = w->N, d = w->d;
    const int64_t hh = t / N, i = t % N;
    const int64_t row_off = ((w->q_head0 + hh) * N + i) * d;
    const int64_t n_vis = w->causal ? i + 1 : N;
    const double* kd = w->kd;
    const double* vd = w->vd;
    double* p = w->work;              /* [N] */
    double* ds = p + N;               /* [N] */
    double* wt = ds + N;              /* [N] */
    double* qrow = wt + N;            /* [d] */
    double* grow = qrow + d;          /* [d]: dO_i */
    double* orow = grow + d;          /* [d] */
    double* qa = orow + d;            /* [d]: |q_i| */
    double* ga = qa + d;              /* [d]: |dO_i| */

    for (int64_t c = 0; c < d; c++) {
        qrow[c] = decode_one(w->q, row_off + c, w->dtype);
        grow[c] = decode_one(w->dout, row_off + c, w->dtype);
        qa[c] = fabs(qrow[c]);
        ga[c] = fabs(grow[c]);
    }
    /* forward row: s_ij, safe softmax p_ij, o_i */
    double m = -INFINITY;
    for (int64_t j = 0; j < n_vis; j++) {
        double dot = 0.0;
        for (int64_t c = 0; c < d; c++)
            dot += qrow[c] * kd[j * d + c];
        p[j] = w->scale * dot;
        if (p[j] > m)
            m = p[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < n_vis; j++) {
        p[j] = exp(p[j] - m);
        l += p[j];
    }
    for (int64_t j = 0; j < n_vis; j++)
        p[j] /= l;
    for (int64_t c = 0; c < d; c++)
        orow[c] = 0.0;
    for (int64_t j = 0; j < n_vis; j++)
        for (int64_t c = 0; c < d; c++)
            orow[c] += p[j] * vd[j * d + c];

    double D = 0.0, A = 0.0, gs = 0.0;
    for (int64_t c = 0; c < d; c++) {
        D += grow[c] * orow[c];
        A += fabs(grow[c] * orow[c]);
        gs += ga[c];
    }
    for (int64_t j = 0; j < n_vis; j++) {
        double dp = 0.0;
        for (int64_t c = 0; c < d; c++)
            dp += grow[c] * vd[j * d + c];
        ds[j] = p[j] * (dp - D);
        wt[j] = fabs(ds[j]) + p[j] * A;
    }

    double* dq = w->dq + row_off;
    for (int64_t c = 0; c < d; c++)
        dq[c] = 0.0;
    for (int64_t j = 0; j < n_vis; j++)
        for (int64_t c = 0; c < d; c++)
            dq[c] += ds[j] * kd[j * d + c];
    for (int64_t c = 0; c < d; c++)
        dq[c] *= w->scale;
    if (w->eq) {
        double* eq = w->eq + row_off;
        for (int64_t c = 0; c < d; c++)
            eq[c] = 0.0;
        for (int64_t j = 0; j < n_vis; j++)
            for (int64_t c = 0; c < d; c++)
                eq[c] += wt[j] * w->ka[j * d + c];
        for (int64_t c = 0; c < d; c++)
            eq[c] *= w->scale;
        double* zq = w->zq + row_off;
        for (int64_t c = 0; c < d; c++)
            zq[c] = 0.0;
        for (int64_t j = 0; j < n_vis; j++) {
            const double z = 1.0 + p[j] * gs;
            for (int64_t c = 0; c < d; c++)
                zq[c] += z * w->ka[j * d + c];
        }
        for (int64_t c = 0; c < d; c++)
            zq[c] *= w->scale;
    }
    for (int64_t j = 0; j < n_vis; j++) {
        const double a = w->scale * ds[j], pj = p[j];
        double* dk = w->dk + j * d;
        double* dv = w->dv + j * d;
        for (int64_t c = 0; c < d; c++) {
            dk[c] += a * qrow[c];
            dv[c] += pj * grow[c];
        }
        if (w->ek) {
            const double b = w->scale * wt[j];
            const double z = w->scale * (1.0 + pj * gs);
            double* ek = w->ek + j * d;
            double* ev = w->ev + j * d;
            double* zk = w->zk + j * d;
            double* zv = w->zv + j * d;
            for (int64_t c = 0; c < d; c++) {
                ek[c] += b * qa[c];
                ev[c] += pj * ga[c];
                zk[c] += z * qa[c];
                zv[c] += ga[c];
            }
        }
    }
}

static void* bwd_worker(void* arg)
{
    bwd_part_t* w = (bwd_part_t*)arg;
    for (int64_t t = w->row_begin; t < w->row_end; t++)
        bwd_row(w, t);
    return NULL;
}

int attn_bwd_ref(const void* q, const void* k, const void* v, const void* dout,
                 double* dq, double* dk, double* dv,
                 double* eq, double* ek, double* ev,
                 double* zq, double* zk, double* zv,
                 int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d,
                 int causal, float scale, int dtype, int num_threads)
{
    int rc = check_args(q, k, v, B, H, H_kv, N, d, causal, scale, dtype);
    if (rc != ATTN_REF_OK)
        return rc;
    if (!dout || !dq || !dk || !dv)
        return ATTN_REF_EINVAL;
    const int with_e = eq != NULL;
    if ((ek != NULL) != with_e || (ev != NULL) != with_e || (zq != NULL) != with_e ||
        (zk != NULL) != with_e || (zv != NULL) != with_e)
        return ATTN_REF_EINVAL;

    const int64_t G = H / H_kv, rows = G * N, nd = N * d;
    if (num_threads <= 0) {
        long n = sysconf(_SC_NPROCESSORS_ONLN);
        num_threads = n > 0 ? (int)n : 1;
    }
    if (num_threads > rows)
        num_threads = (int)rows;
    const int T = num_threads;
    const int n_acc = with_e ? 6 : 2;   /* dk, dv (, ek, ev, zk, zv) per worker */

    double* kd = (double*)malloc((size_t)nd * 3 * sizeof(double));
    double* part = (double*)calloc((size_t)T * n_acc * nd, sizeof(double));
    double* work = (double*)malloc((size_t)T * (3 * N + 5 * d) * sizeof(double));
    bwd_part_t* parts = (bwd_part_t*)calloc((size_t)T, sizeof(bwd_part_t));
    pthread_t* th = (pthread_t*)malloc((size_t)T * sizeof(pthread_t));
    if (!kd || !part || !work || !parts || !th) {
        free(kd); free(part); free(work); free(parts); free(th);
        return ATTN_REF_ENOMEM;
    }
    double* vd = kd + nd;
    double* ka = vd + nd;

    for (int64_t b = 0; b < B; b++)
        for (int64_t hkv = 0; hkv < H_kv; hkv++) {
            const int64_t kv_off = (b * H_kv + hkv) * nd;
            for (int64_t x = 0; x < nd; x++) {
                kd[x] = decode_one(k, kv_off + x, dtype);
                vd[x] = decode_one(v, kv_off + x, dtype);
                ka[x] = fabs(kd[x]);
            }
            memset(part, 0, (size_t)T * n_acc * nd * sizeof(double));
            int started = 0;
            for (int t = 0; t < T; t++) {
                bwd_part_t* w = &parts[t];
                w->q = q; w->dout = dout; w->kd = kd; w->vd = vd; w->ka = ka;
                w->N = N; w->d = d; w->causal = causal;
                w->scale = (double)scale; w->dtype = dtype;
                w->q_head0 = b * H + hkv * G;
                w->row_begin = rows * t / T;
                w->row_end = rows * (t + 1) / T;
                w->dq = dq; w->eq = eq; w->zq = zq;
                double* base = part + (size_t)t * n_acc * nd;
                w->dk = base; w->dv = base + nd;
                w->ek = with_e ? base + 2 * nd : NULL;
                w->ev = with_e ? base + 3 * nd : NULL;
                w->zk = with_e ? base + 4 * nd : NULL;
                w->zv = with_e ? base + 5 * nd : NULL;
                w->work = work + (size_t)t * (3 * N + 5 * d);
            }
            for (int t = 0; t < T; t++) {
                if (pthread_create(&th[t], NULL, bwd_worker, &parts[t]) != 0)
                    break;
                started++;
            }
            for (int t = started; t < T; t++)
                bwd_worker(&parts[t]);   /* workers that could not start run here */
            for (int t = 0; t < started; t++)
                pthread_join(th[t], NULL);
            /* sum the workers' partial dk, dv (, ek, ev, zk, zv) in worker order */
            for (int a = 0; a < n_acc; a++) {
                double* const outs[6] = {dk, dv, ek, ev, zk, zv};
                double* out = outs[a];
                out += kv_off;
                for (int64_t x = 0; x < nd; x++) {
                    double acc = 0.0;
                    for (int t = 0; t < T; t++)
                        acc += part[((size_t)t * n_acc + a) * nd + x];
                    out[x] = acc;
                }
            }
        }
    free(kd); free(part); free(work); free(parts); free(th);
    return ATTN_REF_OK;
}
