/*
 * gsr_oracle.c -- the CPU oracle for the fused fp16 GEMM + scale + ReLU.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library in tiled_dense_gemm_scale_amd/csrc.
 *
 * What it computes (PKUHPC scow-tutorial "Tutorial14: 使用TileLang语言编写
 * attention算子", section 3 "算子介绍", the display formula and its symbol
 * list; the kernel listing of section 2 "编写算子" fixes the dtypes):
 *
 *     C[m,n] = ReLU( alpha * sum_{k<K} A[m,k] * B[k,n] )
 *
 * with A (M x K), B (K x N) and C (M x N) row-major IEEE binary16 arrays,
 * alpha a binary32 scalar, and ReLU(x) = max(x, 0).  The tutorial's kernel
 * applies the scale first and the max second, both in the accumulator
 * precision, and only then narrows to fp16 on the single store.
 *
 * The oracle does every step in IEEE binary64:
 *   1. decode each fp16 input exactly (own bit-level decoder, subnormals
 *      included);
 *   2. s = sum over k in ascending order of a*b -- each product of two fp16
 *      values is exact in binary64 (11-bit x 11-bit significands), so the
 *      only rounding is the fp64 addition, far below the fp16 output ulp;
 *   3. y = (double)alpha * s;
 *   4. r = y if y > 0 else +0.0  (non-positive results, -0 and NaN give +0);
 *   5. C = round-to-nearest-even of r to fp16 (one rounding; r >= 65520
 *      gives +inf).
 * This is the plain triple loop of the TileKernels article (cloud.baidu.com
 * "TileKernels：面向大语言模型的高性能GPU算子库解析", section 五 "开发实践指南",
 * its custom_matmul example: a zeroed accumulator, a k loop of products)
 * followed by the tutorial's epilogue.  Loop order i-k-j is used in the full
 * mode so the j loop vectorises; every output still sums its products in
 * ascending k, exactly as the triple loop does.
 *
 * Readings where the pages are silent: fp64 accumulation (the article's
 * accumulator is a Python float, i.e. binary64), round-to-nearest-even for
 * the fp16 narrowing, +0 for every non-positive result, +inf on overflow.
 *
 * Epilogue variants (the aikraft.ru TileLang guide, section 4 "Слияние
 * эпилогов: GEMM + Bias + GELU": the matmul result gets a bias added and then
 * an exp-based GELU approximation, all before the single store):
 *
 *     C[m,n] = act( alpha * sum_k A[m,k] B[k,n] + bias[n] )
 *
 * with bias an optional fp16 vector over the N output columns and act one of
 * ReLU, GELU or the identity.  GELU is the tanh form
 *     gelu(y) = y/2 * (1 + tanh( sqrt(2/pi) * (y + 0.044715 y^3) )),
 * its tanh taken from exp (the guide names an exponent-based formula).  The
 * guide fixes neither the bias layout nor the GELU constants; the readings
 * are: bias per output column, fp16 like the operands, added in the
 * accumulator precision after the scale; the tanh-form constants above.
 * Activation codes: 0 ReLU, 1 GELU, 2 identity.
 *
 * Compile-time switch ORACLE_MUTANT (default 0) plants one deliberate
 * mistake; it exists only so the pin tests can prove that they catch
 * plausible bugs.  A normal build never defines it.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 2

/* ------------------------------------------------------------------------ */
/* fp16 codec, written from the IEEE 754 binary16 definition:               */
/* 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.                 */
/* ------------------------------------------------------------------------ */

double oracle_fp16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
#if ORACLE_MUTANT == 6
        v = ldexp((double)(1024 + f), -24); /* mistake: implicit 1 on subnormals */
        if (f == 0) v = 0.0;
#else
        v = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
#endif
    } else if (e == 31) {
        v = (f == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + f), e - 25); /* (1.f) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* Round a non-negative integer-plus-fraction value m (exactly representable)
 * to an integer, ties to even. */
static double round_half_even(double m)
{
    double n = floor(m);
    double frac = m - n; /* exact: m and n share the binade */
#if ORACLE_MUTANT == 3
    (void)frac;
    return n; /* mistake: truncation */
#elif ORACLE_MUTANT == 7
    return (frac >= 0.5) ? n + 1.0 : n; /* mistake: ties away from zero */
#else
    if (frac > 0.5) return n + 1.0;
    if (frac < 0.5) return n;
    return (fmod(n, 2.0) == 0.0) ? n : n + 1.0;
#endif
}

uint16_t oracle_f64_to_fp16(double x)
{
    uint16_t sign = 0;
    double ax;
    if (isnan(x)) return 0x7e00;
    if (signbit(x)) sign = 0x8000;
    ax = fabs(x);
    if (ax >= 65520.0) return (uint16_t)(sign | 0x7c00); /* rounds past 65504 */
    if (ax < ldexp(1.0, -14)) {
        /* subnormal range: quantum 2^-24; n == 1024 is the smallest normal,
         * whose bit pattern is exactly 1024 as well */
        double n = round_half_even(ldexp(ax, 24));
        return (uint16_t)(sign | (uint16_t)n);
    } else {
        int E;
        double n;
        int e;
        (void)frexp(ax, &E); /* ax = f * 2^E, f in [0.5, 1) */
        e = E - 1;           /* 2^e <= ax < 2^(e+1), -14 <= e <= 15 */
        n = round_half_even(ldexp(ax, 10 - e)); /* in [1024, 2048] */
        if (n >= 2048.0) {
            n = 1024.0;
            e += 1;
        }
        if (e + 15 >= 31) return (uint16_t)(sign | 0x7c00);
        return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(n - 1024.0));
    }
}

void oracle_decode_array(int64_t n, const uint16_t* in, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_fp16_to_f64(in[i]);
}

void oracle_encode_array(int64_t n, const double* in, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_fp16(in[i]);
}

/* ------------------------------------------------------------------------ */
/* The epilogue of the tutorial's kernel: scale, then ReLU, then narrowing. */
/* ------------------------------------------------------------------------ */

static double scale_relu(double s, float alpha)
{
#if ORACLE_MUTANT == 4
    double r = (s > 0.0) ? s : 0.0; /* mistake: ReLU before the scale */
    double y = (double)alpha * r;
    return (y > 0.0) ? y : 0.0;
#elif ORACLE_MUTANT == 5
    (void)alpha;
    return (s > 0.0) ? s : 0.0; /* mistake: scale dropped */
#else
    double y = (double)alpha * s;
    return (y > 0.0) ? y : 0.0; /* -0 and NaN fall to +0 */
#endif
}

#define ORACLE_ACT_RELU 0
#define ORACLE_ACT_GELU 1
#define ORACLE_ACT_NONE 2

/* GELU, tanh form: y/2 * (1 + tanh(u)), u = sqrt(2/pi) (y + 0.044715 y^3).
 * tanh comes from t = exp(-2|u|) in (0, 1]: tanh(|u|) = (1 - t)/(1 + t), so
 *   1 + tanh(u) = 2/(1 + t)      for u >= 0,
 *   1 + tanh(u) = 2t/(1 + t)     for u <  0,
 * which avoids the cancellation of 1 + tanh(u) when u is very negative. */
double oracle_gelu(double y)
{
    const double c = sqrt(2.0 / 3.14159265358979323846);
#if ORACLE_MUTANT == 11
    const double u = c * y; /* mistake: cubic term dropped */
#else
    const double u = c * (y + 0.044715 * y * y * y);
#endif
    const double t = exp(-2.0 * fabs(u));
    const double one_plus_tanh = (u >= 0.0) ? 2.0 / (1.0 + t) : 2.0 * t / (1.0 + t);
    return 0.5 * y * one_plus_tanh;
}

static double activate(double y, int act)
{
    if (act == ORACLE_ACT_RELU) return (y > 0.0) ? y : 0.0; /* -0 and NaN fall to +0 */
    if (act == ORACLE_ACT_GELU) return oracle_gelu(y);
    return y;
}

/* The general epilogue: act(alpha * s + bias), bias = NULL for none. */
static double epilogue(double s, float alpha, const double* bias_n, int act)
{
    if (!bias_n && act == ORACLE_ACT_RELU) return scale_relu(s, alpha);
#if ORACLE_MUTANT == 9
    (void)bias_n; /* mistake: bias dropped */
    return activate((double)alpha * s, act);
#elif ORACLE_MUTANT == 12
    return activate((double)alpha * s, act) + (bias_n ? *bias_n : 0.0); /* mistake: bias after act */
#else
    return activate((double)alpha * s + (bias_n ? *bias_n : 0.0), act);
#endif
}

/* The bias element that output (m, n) takes. */
static const double* bias_of(const double* biasd, int64_t m, int64_t n)
{
    if (!biasd) return NULL;
#if ORACLE_MUTANT == 10
    (void)n;
    return biasd + m; /* mistake: bias indexed by row */
#else
    (void)m;
    return biasd + n;
#endif
}

/* ------------------------------------------------------------------------ */
/* Full mode: every output.  Rows are split over threads; each output sums  */
/* its products in ascending k.                                             */
/* ------------------------------------------------------------------------ */

typedef struct {
    int64_t M, N, K;
    const double* Ad; /* decoded A, M*K */
    const double* Bd; /* decoded B, K*N */
    float alpha;
    const double* biasd; /* decoded bias, N, or NULL */
    int act;
    uint16_t* C;
    double* R; /* optional: the epilogue's value in fp64 before narrowing */
    int64_t row0, row1;
} full_job;

static void* full_worker(void* p)
{
    full_job* j = (full_job*)p;
    const int64_t N = j->N, K = j->K;
    double* acc = (double*)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
    if (!acc) return (void*)1;
    for (int64_t m = j->row0; m < j->row1; ++m) {
        for (int64_t n = 0; n < N; ++n) acc[n] = 0.0;
#if ORACLE_MUTANT == 1
        for (int64_t k = 0; k + 1 < K; ++k) { /* mistake: last term dropped */
#else
        for (int64_t k = 0; k < K; ++k) {
#endif
#if ORACLE_MUTANT == 2
            const double a = j->Ad[k * j->M + m]; /* mistake: A read column-major */
#else
            const double a = j->Ad[m * K + k];
#endif
            const double* brow = j->Bd + k * N;
#if ORACLE_MUTANT == 8
            for (int64_t n = 0; n < N; ++n) acc[n] = (double)((float)acc[n] + (float)(a * brow[n])); /* mistake: fp32 sum */
#else
            for (int64_t n = 0; n < N; ++n) acc[n] += a * brow[n];
#endif
        }
        for (int64_t n = 0; n < N; ++n) {
            double r = epilogue(acc[n], j->alpha, bias_of(j->biasd, m, n), j->act);
            j->C[m * N + n] = oracle_f64_to_fp16(r);
            if (j->R) j->R[m * N + n] = r;
        }
    }
    free(acc);
    return NULL;
}

/* C = act(alpha * A B + bias) (and, if R != NULL, the fp64 value before
 * narrowing) for all M x N outputs.  bias: N fp16 values or NULL; act: 0 ReLU,
 * 1 GELU, 2 identity.  nthreads <= 0 means 1.  Returns ORACLE_OK or an error
 * code. */
int oracle_gemm_bias_act(int64_t M, int64_t N, int64_t K, const uint16_t* A, const uint16_t* B,
                         const uint16_t* bias, float alpha, int act, uint16_t* C, double* R, int nthreads)
{
    double *Ad = NULL, *Bd = NULL, *biasd = NULL;
    int rc = ORACLE_OK;
    if (M < 0 || N < 0 || K < 0) return ORACLE_EINVAL;
    if (act < ORACLE_ACT_RELU || act > ORACLE_ACT_NONE) return ORACLE_EINVAL;
    if (M == 0 || N == 0) return ORACLE_OK;
    if (!C || (K > 0 && (!A || !B))) return ORACLE_EINVAL;
    if (nthreads <= 0) nthreads = 1;
    if (nthreads > M) nthreads = (int)M;

    Ad = (double*)malloc((size_t)(M * K > 0 ? M * K : 1) * sizeof(double));
    Bd = (double*)malloc((size_t)(K * N > 0 ? K * N : 1) * sizeof(double));
    if (bias) biasd = (double*)malloc((size_t)N * sizeof(double));
    if (!Ad || !Bd || (bias && !biasd)) {
        free(Ad);
        free(Bd);
        free(biasd);
        return ORACLE_ENOMEM;
    }
    oracle_decode_array(M * K, A, Ad);
    oracle_decode_array(K * N, B, Bd);
    if (bias) oracle_decode_array(N, bias, biasd);

    {
        full_job* jobs = (full_job*)calloc((size_t)nthreads, sizeof(full_job));
        pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
        if (!jobs || !th) {
            rc = ORACLE_ENOMEM;
        } else {
            for (int t = 0; t < nthreads; ++t) {
                jobs[t].M = M; jobs[t].N = N; jobs[t].K = K;
                jobs[t].Ad = Ad; jobs[t].Bd = Bd; jobs[t].alpha = alpha;
                jobs[t].biasd = biasd; jobs[t].act = act;
                jobs[t].C = C; jobs[t].R = R;
                jobs[t].row0 = M * t / nthreads;
                jobs[t].row1 = M * (t + 1) / nthreads;
            }
            for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, full_worker, &jobs[t]);
            if (full_worker(&jobs[0]) != NULL) rc = ORACLE_ENOMEM;
            for (int t = 1; t < nthreads; ++t) {
                void* ret = NULL;
                pthread_join(th[t], &ret);
                if (ret != NULL) rc = ORACLE_ENOMEM;
            }
        }
        free(jobs);
        free(th);
    }
    free(Ad);
    free(Bd);
    free(biasd);
    return rc;
}

/* The tutorial's operation: C = ReLU(alpha * A B). */
int oracle_gemm_scale_relu(int64_t M, int64_t N, int64_t K, const uint16_t* A, const uint16_t* B,
                           float alpha, uint16_t* C, double* R, int nthreads)
{
    return oracle_gemm_bias_act(M, N, K, A, B, NULL, alpha, ORACLE_ACT_RELU, C, R, nthreads);
}

/* ------------------------------------------------------------------------ */
/* Point mode: the same definition evaluated one output at a time, reading  */
/* row m of A and column n of B straight from the fp16 arrays.  Used where  */
/* the full product is too large for the host.                              */
/* ------------------------------------------------------------------------ */

typedef struct {
    int64_t M, N, K;
    const uint16_t *A, *B, *bias;
    float alpha;
    int act;
    const int64_t *ms, *ns;
    uint16_t* out;
    double* R;
    int64_t i0, i1;
} point_job;

static void* point_worker(void* p)
{
    point_job* j = (point_job*)p;
    for (int64_t i = j->i0; i < j->i1; ++i) {
        const int64_t m = j->ms[i], n = j->ns[i];
        double s = 0.0;
#if ORACLE_MUTANT == 1
        for (int64_t k = 0; k + 1 < j->K; ++k) {
#else
        for (int64_t k = 0; k < j->K; ++k) {
#endif
#if ORACLE_MUTANT == 2
            const double a = oracle_fp16_to_f64(j->A[k * j->M + m]);
#else
            const double a = oracle_fp16_to_f64(j->A[m * j->K + k]);
#endif
            const double b = oracle_fp16_to_f64(j->B[k * j->N + n]);
#if ORACLE_MUTANT == 8
            s = (double)((float)s + (float)(a * b));
#else
            s += a * b;
#endif
        }
        {
            double bd = 0.0;
            const double* bp = NULL;
            if (j->bias) {
#if ORACLE_MUTANT == 10
                bd = oracle_fp16_to_f64(j->bias[m]); /* mistake: bias indexed by row */
#else
                bd = oracle_fp16_to_f64(j->bias[n]);
#endif
                bp = &bd;
            }
            double r = epilogue(s, j->alpha, bp, j->act);
            j->out[i] = oracle_f64_to_fp16(r);
            if (j->R) j->R[i] = r;
        }
    }
    return NULL;
}

/* Outputs C[ms[i], ns[i]] of act(alpha * A B + bias) for i < npts.  Indices
 * must lie in [0,M) x [0,N); bias (N values) may be NULL. */
int oracle_gemm_bias_act_points(int64_t M, int64_t N, int64_t K, const uint16_t* A, const uint16_t* B,
                                const uint16_t* bias, float alpha, int act, int64_t npts, const int64_t* ms,
                                const int64_t* ns, uint16_t* out, double* R, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || npts < 0) return ORACLE_EINVAL;
    if (act < ORACLE_ACT_RELU || act > ORACLE_ACT_NONE) return ORACLE_EINVAL;
    if (npts == 0) return ORACLE_OK;
    if (!ms || !ns || !out || (K > 0 && (!A || !B))) return ORACLE_EINVAL;
    for (int64_t i = 0; i < npts; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N) return ORACLE_EINVAL;
    if (nthreads <= 0) nthreads = 1;
    if (nthreads > npts) nthreads = (int)npts;
    {
        point_job* jobs = (point_job*)calloc((size_t)nthreads, sizeof(point_job));
        pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
        if (!jobs || !th) {
            free(jobs);
            free(th);
            return ORACLE_ENOMEM;
        }
        for (int t = 0; t < nthreads; ++t) {
            jobs[t].M = M; jobs[t].N = N; jobs[t].K = K;
            jobs[t].A = A; jobs[t].B = B; jobs[t].bias = bias; jobs[t].alpha = alpha; jobs[t].act = act;
            jobs[t].ms = ms; jobs[t].ns = ns; jobs[t].out = out; jobs[t].R = R;
            jobs[t].i0 = npts * t / nthreads;
            jobs[t].i1 = npts * (t + 1) / nthreads;
        }
        for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, point_worker, &jobs[t]);
        point_worker(&jobs[0]);
        for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
        free(jobs);
        free(th);
    }
    return ORACLE_OK;
}

/* The tutorial's operation at chosen outputs. */
int oracle_gemm_scale_relu_points(int64_t M, int64_t N, int64_t K, const uint16_t* A, const uint16_t* B,
                                  float alpha, int64_t npts, const int64_t* ms, const int64_t* ns,
                                  uint16_t* out, double* R, int nthreads)
{
    return oracle_gemm_bias_act_points(M, N, K, A, B, NULL, alpha, ORACLE_ACT_RELU, npts, ms, ns, out, R, nthreads);
}

int oracle_mutant_id(void) { return ORACLE_MUTANT; }
