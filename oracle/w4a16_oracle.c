/*
 * w4a16_oracle.c -- CPU oracle for the fused W4A16 dequantize-GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  The
 * product path never calls it, and it includes nothing from the product
 * sources (no shared headers, helpers, tables or constants).
 *
 * What it computes, written out as the plain definition:
 *
 *   q[k][n]   = nibble (k mod 8) of qweight[k/8][n], least-significant nibble
 *               first.  Page "W4A16 GEMM 算子浅析" (nxmr.cn), section
 *               "Marlin 与 CUTLASS 中的寄存器解包黑魔法": one 32-bit word holds
 *               eight independent 4-bit weights.  The order of the eight
 *               inside the word is not stated; this file reads it as
 *               nibble i = bits 4i..4i+3 = k index 8*(k/8)+i.
 *   g         = floor(k / G); z[g][n] = zeros[g][n] (asymmetric) or 8
 *               (symmetric).
 *   deq[k][n] = RNE_dtype( (q[k][n] - z[g][n]) * s[g][n] ).
 *               Page "W4A16 GEMM 算子浅析", section "计算流水线的核心哲学"
 *               (pipeline diagram, register dequant step: weight minus zero,
 *               times scale); page "量化开销对比" (laojiahuo2003.github.io),
 *               section 2, W = s_w (W^q - z_w).  The product is exact in
 *               fp64 (an integer of at most 4 bits times a significand of at
 *               most 11 bits), so the only rounding is the single
 *               round-to-nearest-even into the activation dtype.
 *   Y[m][n]   = sum over k of X[m][k] * deq[k][n], accumulated in fp64 in
 *               increasing k.  Page "量化开销对比", section 6.2: the group
 *               scale changes along the reduction index, so it multiplies
 *               each weight before the sum.
 *   B[m][n]   = sum over k of |X[m][k]| * |deq[k][n]|, the denominator of the
 *               error bound a floating-point dot product is judged by.
 *   Yx[m][n]  = (diagnostic) the same sum with the unrounded (q - z) * s.
 *
 * Every product X*deq is exact in fp64 (11+11 significant bits at most), so
 * Y differs from the exact rational sum by at most about K * 2^-53 * B.
 *
 * Epilogue (oracle_epilogue), the output-side steps the fused kernel may run
 * before its single store.  Page "量化开销对比", sections 6.2 (after the k
 * loop the accumulator is multiplied by a scale, the bias is added and the
 * result written), 6.6 (dequant, GEMM, scale and bias, plus residual or
 * activation, in one kernel) and 6.7 (a per-channel scale multiplies the
 * output in the epilogue).  Read, in this order, each step optional:
 *   t = Y[m][n] * c[n] + b[n];   u = act(t);   y = u + a[m][n]  or  u * a[m][n]
 * with act = identity, ReLU max(t, 0) or SiLU t / (1 + exp(-t)), all in fp64.
 * Its error-bound denominator carries B through the same steps:
 *   Bo = |a| * L * (|c| * B + |b|)  (multiply)  or  L * (|c| * B + |b|) + |a|  (add),
 * L = 1 (identity, ReLU) or 1.1 (SiLU, whose slope stays below 1.1), so that
 * |y| <= Bo and the identity epilogue gives Bo = B.
 *
 * Layouts (all row-major, the canonical tensors of the library boundary):
 *   X        uint16 bit patterns [M][K] (fp16 or bf16)
 *   qweight  uint32 [K/8][N]
 *   scales   uint16 bit patterns [K/G][N] (same dtype as X)
 *   zeros    uint8 [K/G][N], values 0..15; ignored when sym != 0
 *
 * Build: gcc -O2 -ffp-contract=off -shared -fPIC -pthread w4a16_oracle.c -lm
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_VERSION 1

/* Activation dtype codes used by this file only. */
enum { ORACLE_F16 = 0, ORACLE_BF16 = 1 };

int oracle_version(void) { return ORACLE_VERSION; }

/* ---------------------------------------------------------------------- */
/* IEEE binary16 and bfloat16 <-> double, by their field definitions.      */
/* ---------------------------------------------------------------------- */

double oracle_f16_to_double(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

double oracle_bf16_to_double(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 7) & 255;
    int m = h & 127;
    double v;
    if (e == 0)
        v = ldexp((double)m, -133);                /* subnormal: m * 2^-133 */
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + m), e - 134);     /* (1 + m/2^7) * 2^(e-127) */
    return sign ? -v : v;
}

/*
 * Round a double to the nearest binary16 value, ties to even, and return its
 * bit pattern.  The spacing of binary16 values in [2^E, 2^(E+1)) is
 * 2^(E-10); below 2^-14 it stays 2^-24.  nearbyint() rounds ties to even in
 * the default rounding mode.
 */
uint16_t oracle_round_f16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return 0x7E00;
    if (isinf(a))
        return sign | 0x7C00;
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2);                 /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;
    if (E < -14)
        E = -14;
    double ulp = ldexp(1.0, E - 10);
    double r = nearbyint(a / ulp) * ulp;
    if (r >= 65536.0)
        return sign | 0x7C00;      /* rounds past the largest finite, 65504 */
    if (r < ldexp(1.0, -14))
        return sign | (uint16_t)ldexp(r, 24);   /* subnormal field = r / 2^-24 */
    frexp(r, &e2);
    E = e2 - 1;
    uint16_t field_e = (uint16_t)(E + 15);
    uint16_t field_m = (uint16_t)(ldexp(r, 10 - E) - 1024.0);
    return sign | (uint16_t)(field_e << 10) | field_m;
}

/* Same for bfloat16: spacing 2^(E-7) in [2^E, 2^(E+1)), 2^-133 below 2^-126. */
uint16_t oracle_round_bf16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return 0x7FC0;
    if (isinf(a))
        return sign | 0x7F80;
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2);
    int E = e2 - 1;
    if (E < -126)
        E = -126;
    double ulp = ldexp(1.0, E - 7);
    double r = nearbyint(a / ulp) * ulp;
    if (r >= ldexp(1.0, 128))
        return sign | 0x7F80;
    if (r < ldexp(1.0, -126))
        return sign | (uint16_t)ldexp(r, 133);
    frexp(r, &e2);
    E = e2 - 1;
    uint16_t field_e = (uint16_t)(E + 127);
    uint16_t field_m = (uint16_t)(ldexp(r, 7 - E) - 128.0);
    return sign | (uint16_t)(field_e << 7) | field_m;
}

static double to_double(uint16_t bits, int dtype)
{
    return dtype == ORACLE_BF16 ? oracle_bf16_to_double(bits) : oracle_f16_to_double(bits);
}

static uint16_t round_to(double v, int dtype)
{
    return dtype == ORACLE_BF16 ? oracle_round_bf16(v) : oracle_round_f16(v);
}

/* ---------------------------------------------------------------------- */
/* The method's steps.                                                     */
/* ---------------------------------------------------------------------- */

static int check_shape(int64_t K, int64_t N, int64_t G, int dtype)
{
    if (K <= 0 || N <= 0 || G <= 0)
        return 1;
    if (K % 8 != 0 || K % G != 0)
        return 1;
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16)
        return 1;
    return 0;
}

/* q[k][n]: nibble k%8 of word qweight[k/8][n], least significant first. */
static inline int nibble_at(const uint32_t *qweight, int64_t N, int64_t k, int64_t n)
{
    uint32_t word = qweight[(k / 8) * N + n];
    return (int)((word >> (4 * (k % 8))) & 0xFu);
}

static inline int zero_at(const uint8_t *zeros, int sym, int64_t N, int64_t g, int64_t n)
{
    return sym ? 8 : (int)zeros[g * N + n];
}

/* Exact (q - z) * s for one weight, in fp64. */
static inline double dequant_exact(const uint32_t *qweight, const uint16_t *scales,
                                   const uint8_t *zeros, int64_t N, int64_t G,
                                   int dtype, int sym, int64_t k, int64_t n)
{
    int64_t g = k / G;
    int q = nibble_at(qweight, N, k, n);
    int z = zero_at(zeros, sym, N, g, n);
    double s = to_double(scales[g * N + n], dtype);
    return (double)(q - z) * s;
}

/* Writes q[K][N] (uint8).  Returns 0, or 1 on a bad shape. */
int oracle_unpack(const uint32_t *qweight, int64_t K, int64_t N, uint8_t *q)
{
    if (K <= 0 || N <= 0 || K % 8 != 0)
        return 1;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            q[k * N + n] = (uint8_t)nibble_at(qweight, N, k, n);
    return 0;
}

/*
 * Writes deq_bits[K][N] (the dtype's bit pattern of RNE((q - z) * s)) and,
 * when deq_exact is not NULL, the unrounded (q - z) * s in fp64.
 */
int oracle_dequant(const uint32_t *qweight, const uint16_t *scales, const uint8_t *zeros,
                   int64_t K, int64_t N, int64_t G, int dtype, int sym,
                   uint16_t *deq_bits, double *deq_exact)
{
    if (check_shape(K, N, G, dtype) || (!sym && zeros == NULL))
        return 1;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            double e = dequant_exact(qweight, scales, zeros, N, G, dtype, sym, k, n);
            deq_bits[k * N + n] = round_to(e, dtype);
            if (deq_exact)
                deq_exact[k * N + n] = e;
        }
    return 0;
}

/* Scale-only variant: RNE((q - z) * s) for given arrays of q, z and scale bits. */
int oracle_dequant_values(const uint8_t *q, const uint8_t *z, const uint16_t *s_bits,
                          int64_t count, int dtype, uint16_t *deq_bits)
{
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16)
        return 1;
    for (int64_t i = 0; i < count; ++i)
        deq_bits[i] = round_to((double)((int)q[i] - (int)z[i]) * to_double(s_bits[i], dtype), dtype);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* GEMM: Y = X . deq, fp64 accumulation, threads over column ranges.       */
/* ---------------------------------------------------------------------- */

typedef struct {
    const uint16_t *X;
    const double *Xd;           /* X converted to fp64, [M][K] */
    const uint32_t *qweight;
    const uint16_t *scales;
    const uint8_t *zeros;
    int64_t M, N, K, G;
    int dtype, sym;
    double *Y, *Bnd, *Yx;       /* [M][N]; Bnd and Yx may be NULL */
    /* full-matrix mode: column range [n0, n1) */
    int64_t n0, n1;
    /* sampled mode: pairs [p0, p1) of (ms[i], ns[i]) */
    const int64_t *ms, *ns;
    int64_t p0, p1;
    int status;
} job_t;

static void *gemm_columns(void *arg)
{
    job_t *j = (job_t *)arg;
    double *col = (double *)malloc((size_t)j->K * sizeof(double));
    double *colx = (double *)malloc((size_t)j->K * sizeof(double));
    if (!col || !colx) {
        j->status = 2;
        free(col);
        free(colx);
        return NULL;
    }
    for (int64_t n = j->n0; n < j->n1; ++n) {
        /* deq[:, n] -- a function of (k, n) only, evaluated once per column */
        for (int64_t k = 0; k < j->K; ++k) {
            double e = dequant_exact(j->qweight, j->scales, j->zeros, j->N, j->G,
                                     j->dtype, j->sym, k, n);
            colx[k] = e;
            col[k] = to_double(round_to(e, j->dtype), j->dtype);
        }
        for (int64_t m = 0; m < j->M; ++m) {
            const double *x = j->Xd + m * j->K;
            double acc = 0.0, bnd = 0.0, accx = 0.0;
            for (int64_t k = 0; k < j->K; ++k) {
                acc += x[k] * col[k];
                bnd += fabs(x[k]) * fabs(col[k]);
                accx += x[k] * colx[k];
            }
            j->Y[m * j->N + n] = acc;
            if (j->Bnd)
                j->Bnd[m * j->N + n] = bnd;
            if (j->Yx)
                j->Yx[m * j->N + n] = accx;
        }
    }
    free(col);
    free(colx);
    return NULL;
}

static void *gemm_pairs(void *arg)
{
    job_t *j = (job_t *)arg;
    for (int64_t i = j->p0; i < j->p1; ++i) {
        int64_t m = j->ms[i], n = j->ns[i];
        const uint16_t *x = j->X + m * j->K;
        double acc = 0.0, bnd = 0.0;
        for (int64_t k = 0; k < j->K; ++k) {
            double e = dequant_exact(j->qweight, j->scales, j->zeros, j->N, j->G,
                                     j->dtype, j->sym, k, n);
            double w = to_double(round_to(e, j->dtype), j->dtype);
            double xv = to_double(x[k], j->dtype);
            acc += xv * w;
            bnd += fabs(xv) * fabs(w);
        }
        j->Y[i] = acc;
        j->Bnd[i] = bnd;
    }
    return NULL;
}

static int resolve_threads(int nthreads, int64_t work)
{
    if (nthreads <= 0) {
        long c = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = c > 0 ? (int)c : 1;
    }
    if (nthreads > 256)
        nthreads = 256;
    if ((int64_t)nthreads > work)
        nthreads = (int)(work > 0 ? work : 1);
    return nthreads;
}

static int run_jobs(job_t *jobs, int nt, void *(*fn)(void *))
{
    pthread_t tid[256];
    int started[256];
    for (int t = 0; t < nt; ++t)
        started[t] = pthread_create(&tid[t], NULL, fn, &jobs[t]) == 0;
    for (int t = 0; t < nt; ++t) {
        if (started[t])
            pthread_join(tid[t], NULL);
        else
            fn(&jobs[t]);
    }
    for (int t = 0; t < nt; ++t)
        if (jobs[t].status)
            return jobs[t].status;
    return 0;
}

/*
 * Full product.  Y[M][N] (required), Bnd[M][N] and Yx[M][N] (optional).
 * nthreads <= 0 uses every online CPU.  Returns 0, 1 on a bad shape, 2 on
 * an allocation failure.
 */
int oracle_gemm(const uint16_t *X, const uint32_t *qweight, const uint16_t *scales,
                const uint8_t *zeros, int64_t M, int64_t N, int64_t K, int64_t G,
                int dtype, int sym, double *Y, double *Bnd, double *Yx, int nthreads)
{
    if (M <= 0 || check_shape(K, N, G, dtype) || (!sym && zeros == NULL) || Y == NULL)
        return 1;
    double *Xd = (double *)malloc((size_t)(M * K) * sizeof(double));
    if (!Xd)
        return 2;
    for (int64_t i = 0; i < M * K; ++i)
        Xd[i] = to_double(X[i], dtype);
    int nt = resolve_threads(nthreads, N);
    job_t jobs[256];
    for (int t = 0; t < nt; ++t) {
        job_t j = {X, Xd, qweight, scales, zeros, M, N, K, G, dtype, sym, Y, Bnd, Yx,
                   N * t / nt, N * (t + 1) / nt, NULL, NULL, 0, 0, 0};
        jobs[t] = j;
    }
    int rc = run_jobs(jobs, nt, gemm_columns);
    free(Xd);
    return rc;
}

/*
 * Sampled product: Y[i] and Bnd[i] for output element (ms[i], ns[i]),
 * i < count.  Each element is computed on its own from the definition.
 */
int oracle_gemm_at(const uint16_t *X, const uint32_t *qweight, const uint16_t *scales,
                   const uint8_t *zeros, int64_t M, int64_t N, int64_t K, int64_t G,
                   int dtype, int sym, const int64_t *ms, const int64_t *ns, int64_t count,
                   double *Y, double *Bnd, int nthreads)
{
    if (M <= 0 || check_shape(K, N, G, dtype) || (!sym && zeros == NULL) || !Y || !Bnd)
        return 1;
    for (int64_t i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N)
            return 1;
    int nt = resolve_threads(nthreads, count);
    job_t jobs[256];
    for (int t = 0; t < nt; ++t) {
        job_t j = {X, NULL, qweight, scales, zeros, M, N, K, G, dtype, sym, Y, Bnd, NULL,
                   0, 0, ms, ns, count * t / nt, count * (t + 1) / nt, 0};
        jobs[t] = j;
    }
    return run_jobs(jobs, nt, gemm_pairs);
}

/* ------------------------------------------------------------------------ */
/* Epilogue on n_el output elements (ms[i], ns[i]) of an M x N output:      */
/* Y, B hold the accumulator and its bound for those elements (as returned  */
/* by oracle_gemm or oracle_gemm_at).  col_scale: fp64 [N] or NULL; bias:   */
/* bit patterns [N] or NULL; aux: bit patterns [M][N] or NULL.              */
/* act: 0 identity, 1 ReLU, 2 SiLU.  aux_op: 0 add, 1 multiply.             */
/* ------------------------------------------------------------------------ */
static double act_apply(double t, int act)
{
    if (act == 1) return t > 0.0 ? t : 0.0;
    if (act == 2) return t / (1.0 + exp(-t));
    return t;
}

int oracle_epilogue(const double *Y, const double *B, const int64_t *ms, const int64_t *ns,
                    int64_t n_el, int64_t M, int64_t N, const double *col_scale,
                    const uint16_t *bias, const uint16_t *aux, int dtype, int act, int aux_op,
                    double *Yout, double *Bout)
{
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return 1;
    if (act < 0 || act > 2 || aux_op < 0 || aux_op > 1) return 1;
    const double L = act == 2 ? 1.1 : 1.0;
    for (int64_t i = 0; i < n_el; ++i) {
        const int64_t m = ms[i], n = ns[i];
        if (m < 0 || m >= M || n < 0 || n >= N) return 1;
        const double c = col_scale ? col_scale[n] : 1.0;
        const double b = bias ? to_double(bias[n], dtype) : 0.0;
        double t = Y[i] * c + b;
        double bt = fabs(c) * B[i] + fabs(b);
        double y = act_apply(t, act);
        double by = L * bt;
        if (aux) {
            const double a = to_double(aux[m * N + n], dtype);
            if (aux_op == 1) {
                y = y * a;
                by = fabs(a) * by;
            } else {
                y = y + a;
                by = by + fabs(a);
            }
        }
        Yout[i] = y;
        Bout[i] = by;
    }
    return 0;
}
