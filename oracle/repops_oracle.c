/*
 * repops_oracle.c -- plain, slow CPU oracle for the reproducible FP32 matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load, link or
 * call this file: it exists so that tests, the smoke check and the CPU
 * baseline leg of the benchmark can compare the GPU library against an
 * obviously correct definition.  It shares no code, header or constant with
 * the GPU library.
 *
 * What it computes (Verde and RepOps article, section 3.2 "RepOps design
 * principles", item 2, the matrix-multiplication example): every output
 * C(i, j) is the inner product of row i of op(A) and column j of op(B),
 * accumulated one term at a time in ascending k and in no other order, from
 * a running sum that starts at zero; the (i, j) themselves may be computed
 * in any order.  In this file's notation, with x_k = op(A)(i, k) and
 * y_k = op(B)(k, j):
 *
 *     s_0 = +0,   s_{k+1} = RN(s_k + RN(x_k * y_k)),   C(i, j) = s_K
 *
 * Readings taken here where the pages are open:
 *   - the multiply and the add are two separately rounded binary32
 *     operations: the Zoo chain-soundness spec ("Detailed proof:
 *     deterministic ordering", paragraph "Determinism of left-fold") pins
 *     round-to-nearest-even and switches fused multiply-add off in
 *     deterministic mode;
 *   - IEEE-754 binary32 with gradual underflow (the RepOps article, section
 *     3.3, requires IEEE-754 compliant hardware), so no flush-to-zero and no
 *     denormals-are-zero;
 *   - the running sum starts at +0.0f and the first product is added to it;
 *   - op(A)(i,k) = A[i*a_rs + k*a_cs] when trans_a == 0, else
 *     A[k*a_rs + i*a_cs]; op(B)(k,j) likewise with trans_b.  Strides are in
 *     elements and describe the stored matrix (the article, section 3.1,
 *     names tensor strides as a source of nondeterminism: here they only
 *     change where a value is read from, never the arithmetic).
 *
 * Threads split the i loop statically.  i is a free dimension, so the thread
 * count never changes a bit of the output.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math
 *        -fexcess-precision=standard -fPIC -shared -pthread
 */
#define _GNU_SOURCE
#include <fenv.h>
#include <float.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <xmmintrin.h>

#if !defined(FLT_EVAL_METHOD) || FLT_EVAL_METHOD != 0
#error "binary32 expressions must be evaluated in binary32 (no x87 excess precision)"
#endif

#pragma STDC FP_CONTRACT OFF

/* Bits of the environment check returned by repops_oracle_env_status(). */
#define ORACLE_ENV_ROUNDING 1 /* rounding mode is not round-to-nearest-even */
#define ORACLE_ENV_FTZ 2      /* MXCSR flush-to-zero is on */
#define ORACLE_ENV_DAZ 4      /* MXCSR denormals-are-zero is on */

int repops_oracle_env_status(void)
{
    int bad = 0;
    unsigned csr = _mm_getcsr();
    if (fegetround() != FE_TONEAREST) bad |= ORACLE_ENV_ROUNDING;
    if (csr & (1u << 15)) bad |= ORACLE_ENV_FTZ;
    if (csr & (1u << 6)) bad |= ORACLE_ENV_DAZ;
    return bad;
}

typedef struct {
    const float *A;
    int64_t a_rs, a_cs;
    const float *B;
    int64_t b_rs, b_cs;
    float *C;
    int64_t c_rs, c_cs;
    int64_t M, N, K;
    int trans_a, trans_b;
    /* entries mode: when ii != NULL, compute out[e] for e in [lo, hi) */
    const int64_t *ii, *jj;
    float *out;
    int64_t lo, hi;
} oracle_job;

/*
 * s_K of the recurrence above for one output: x points at x_0 and x_k sits at
 * x[k * xs]; likewise y_k at y[k * ys].  Each of the two statements in the
 * loop body is one binary32 operation, rounded on its own (FP_CONTRACT is
 * off and FLT_EVAL_METHOD is 0).
 */
static float fixed_order_entry(const float *x, int64_t xs, const float *y, int64_t ys,
                               int64_t K)
{
    float s = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        const float prod = x[k * xs] * y[k * ys]; /* RN(x_k * y_k) */
        s = s + prod;                             /* RN(s_k + prod) */
    }
    return s;
}

/* Where row i of op(A) starts, and its step along k, in elements. */
static const float *op_a_row(const oracle_job *t, int64_t i, int64_t *step)
{
    if (t->trans_a) { *step = t->a_rs; return t->A + i * t->a_cs; }
    *step = t->a_cs; return t->A + i * t->a_rs;
}

/* Where column j of op(B) starts, and its step along k, in elements. */
static const float *op_b_col(const oracle_job *t, int64_t j, int64_t *step)
{
    if (t->trans_b) { *step = t->b_cs; return t->B + j * t->b_rs; }
    *step = t->b_rs; return t->B + j * t->b_cs;
}

static float entry_of(const oracle_job *t, int64_t i, int64_t j)
{
    int64_t xs, ys;
    const float *x = op_a_row(t, i, &xs);
    const float *y = op_b_col(t, j, &ys);
    return fixed_order_entry(x, xs, y, ys, t->K);
}

/* A thread's share: rows [lo, hi) of C, or entries [lo, hi) in entries mode. */
static void *work_range(void *arg)
{
    const oracle_job *t = (const oracle_job *)arg;
    if (t->ii) {
        for (int64_t e = t->lo; e < t->hi; ++e) t->out[e] = entry_of(t, t->ii[e], t->jj[e]);
        return NULL;
    }
    for (int64_t i = t->lo; i < t->hi; ++i)
        for (int64_t j = 0; j < t->N; ++j) t->C[i * t->c_rs + j * t->c_cs] = entry_of(t, i, j);
    return NULL;
}

/* Split [0, total) statically over nthreads and run each part. */
static int run_split(oracle_job base, int64_t total, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > total) nthreads = (int)(total > 0 ? total : 1);
    pthread_t tid[256];
    oracle_job jobs[256];
    int started = 0, rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].lo = total * t / nthreads;
        jobs[t].hi = total * (t + 1) / nthreads;
    }
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tid[t], NULL, work_range, &jobs[t]) != 0) {
            rc = -3;
            break;
        }
        ++started;
    }
    work_range(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(tid[t], NULL);
    if (rc != 0) { /* finish the parts whose threads did not start */
        for (int t = started + 1; t < nthreads; ++t) work_range(&jobs[t]);
    }
    return 0;
}

/*
 * Full product: C(i,j) for all 0 <= i < M, 0 <= j < N, written through
 * (c_rs, c_cs).  Returns 0, or -1 for negative sizes, -2 for an environment
 * that is not round-to-nearest-even with gradual underflow.
 */
int repops_oracle_matmul_f32(const float *A, int64_t a_rs, int64_t a_cs,
                             const float *B, int64_t b_rs, int64_t b_cs,
                             float *C, int64_t c_rs, int64_t c_cs,
                             int64_t M, int64_t N, int64_t K,
                             int trans_a, int trans_b, int nthreads)
{
    if (M < 0 || N < 0 || K < 0) return -1;
    if (repops_oracle_env_status() != 0) return -2;
    if (M == 0 || N == 0) return 0;
    oracle_job base = {A, a_rs, a_cs, B, b_rs, b_cs, C, c_rs, c_cs, M, N, K,
                       trans_a, trans_b, NULL, NULL, NULL, 0, 0};
    return run_split(base, M, nthreads);
}

/*
 * Selected entries: out[e] = C(ii[e], jj[e]) for 0 <= e < count, for checks
 * at sizes where the full product is too slow on the CPU.
 */
int repops_oracle_entries_f32(const float *A, int64_t a_rs, int64_t a_cs,
                              const float *B, int64_t b_rs, int64_t b_cs,
                              int64_t M, int64_t N, int64_t K,
                              int trans_a, int trans_b,
                              const int64_t *ii, const int64_t *jj, int64_t count,
                              float *out, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || count < 0) return -1;
    if (repops_oracle_env_status() != 0) return -2;
    for (int64_t e = 0; e < count; ++e)
        if (ii[e] < 0 || ii[e] >= M || jj[e] < 0 || jj[e] >= N) return -1;
    if (count == 0) return 0;
    oracle_job base = {A, a_rs, a_cs, B, b_rs, b_cs, NULL, 0, 0, M, N, K,
                       trans_a, trans_b, ii, jj, out, 0, 0};
    return run_split(base, count, nthreads);
}

/*
 * Fixed-order average of k contributor gradients and the SGD step, element
 * by element (Zoo Per-LLM Chain Soundness, "Detailed proof: deterministic
 * ordering": paragraphs "Ordering subroutine", "Determinism of left-fold"
 * and "Update step"):
 *
 *     S     = (((g_0 + g_1) + g_2) + ...) + g_{k-1}   left fold, in the given
 *                                                      (canonical) order
 *     gbar  = (1/k) * S
 *     theta = theta - eta * gbar
 *
 * Readings: every operation is a separately rounded binary32 operation
 * (round-to-nearest-even, no fused multiply-add, as the spec's kernel
 * manifest pins); "(1/k) *" is the binary32 quotient 1/k, rounded once, times
 * S; the fold starts from g_0 itself (no +0 in front).  grads[c] points at d
 * floats of contributor c, already in fold order.  theta_out may equal
 * theta_in; gbar_out may be NULL.  Returns 0, -1 for bad sizes, -2 for a
 * floating-point environment that is not RNE with gradual underflow.
 */
int repops_oracle_fold_mean_sgd_f32(const float *const *grads, int64_t k, int64_t d, float eta,
                                    const float *theta_in, float *theta_out, float *gbar_out)
{
    if (k < 1 || d < 0) return -1;
    if (repops_oracle_env_status() != 0) return -2;
    const float inv_k = 1.0f / (float)k;
    for (int64_t e = 0; e < d; ++e) {
        float s = grads[0][e];
        for (int64_t c = 1; c < k; ++c) s = s + grads[c][e];
        const float gbar = inv_k * s;
        if (gbar_out) gbar_out[e] = gbar;
        const float step = eta * gbar;
        theta_out[e] = theta_in[e] - step;
    }
    return 0;
}

/*
 * Batched product with an optional bias, for each b in [0, batch):
 *   C_b(i, j) = RN(S_b(i, j) + bias_b(j))   (or S_b(i, j) without a bias)
 * where S_b(i, j) is the fixed-order sum above over op(A_b) and op(B_b), and
 * X_b starts at X + b * x_bs.  Batch is one more free dimension (the
 * Verde and RepOps article, section 3.2 item 1: dimensions that do not
 * affect the order are parallelised freely).  Reading: the bias is one more
 * separately rounded add after the whole sum (y = xW + b, with the sum
 * complete before the bias is added); bias_b(j) = bias[b * bias_bs + j * bias_s].
 * Returns 0, -1 for bad sizes, -2 for a bad floating-point environment.
 */
int repops_oracle_matmul_batched_f32(const float *A, int64_t a_bs, int64_t a_rs, int64_t a_cs,
                                     const float *B, int64_t b_bs, int64_t b_rs, int64_t b_cs,
                                     float *C, int64_t c_bs, int64_t c_rs, int64_t c_cs,
                                     int64_t M, int64_t N, int64_t K, int64_t batch,
                                     int trans_a, int trans_b,
                                     const float *bias, int64_t bias_bs, int64_t bias_s,
                                     int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || batch < 0) return -1;
    if (repops_oracle_env_status() != 0) return -2;
    for (int64_t b = 0; b < batch; ++b) {
        float *Cb = C + b * c_bs;
        int rc = repops_oracle_matmul_f32(A + b * a_bs, a_rs, a_cs, B + b * b_bs, b_rs, b_cs,
                                          Cb, c_rs, c_cs, M, N, K, trans_a, trans_b, nthreads);
        if (rc != 0) return rc;
        if (bias) {
            for (int64_t i = 0; i < M; ++i)
                for (int64_t j = 0; j < N; ++j) {
                    const float s = Cb[i * c_rs + j * c_cs];
                    Cb[i * c_rs + j * c_cs] = s + bias[b * bias_bs + j * bias_s];
                }
        }
    }
    return 0;
}

/* ---- Other RepOps operators: ERF, GeLU, LayerNorm ------------------------
 * The Verde and RepOps article (section 4.3) names LayerNorm, GeLU and ERF as
 * the operators behind DistilBERT's higher overhead, without formulas.  Each
 * function below fixes one sequence of binary32 operations (every +, -, *, /
 * and sqrt rounded to nearest even on its own, IEEE gradual underflow), so the
 * result is one bit pattern on any IEEE machine.
 */

/* erf, in two pieces split at |x| = 1.
 *
 * |x| < 1: the Maclaurin series erf x = (2/sqrt pi) sum_n (-1)^n x^(2n+1) /
 * (n! (2n+1)), truncated after n = 10 (the first omitted term is below
 * 1.3e-9 there).  Coefficient n is that exact value rounded to binary32 (the
 * decimals below carry 22 digits of it).  Evaluation: w = x*x; by Horner's
 * rule in w from c10 down, s = c10; s = s*w + c9; ...; s = s*w + c0; then
 * erf x = s * x.
 *
 * |x| >= 1 (and NaN): Abramowitz and Stegun, Handbook of Mathematical
 * Functions (1964), formula 7.1.28: for y >= 0,
 *     erf y = 1 - 1 / (1 + a1 y + a2 y^2 + a3 y^3 + a4 y^4 + a5 y^5 + a6 y^6)^16
 * with absolute error at most 3e-7 in exact arithmetic; the coefficients are
 * the handbook's decimals rounded to binary32.  Evaluation: y = |x|; p = a6;
 * p = p*y + a5; ...; p = p*y + a1; p = p*y + 1; q = p^16 by four squarings;
 * r = 1/q; e = 1 - r; erf x = e with the sign of x.
 * (Below |x| = 1 the 16th power would magnify the rounding of p to about
 * 2e-6; the series keeps the binary32 result within a few units of the last
 * place there.) */
static const float ERF_SERIES[11] = {
    1.128379167095512573896e+0f, -3.761263890318375246321e-1f, 1.128379167095512573896e-1f,
    -2.686617064513125175943e-2f, 5.223977625442187842112e-3f, -8.548327023450852832547e-4f,
    1.205533298178966425103e-4f, -1.492565035840625097746e-5f, 1.646211436588924740161e-6f,
    -1.636584469123492431739e-7f, 1.480719281587921723955e-8f};
static const float AS_7128[6] = {0.0705230784f, 0.0422820123f, 0.0092705272f,
                                 0.0001520143f, 0.0002765672f, 0.0000430638f};

static float erf_piecewise(float x)
{
    const float y = fabsf(x);
    if (y < 1.0f) {
        const float w = x * x;
        float s = ERF_SERIES[10];
        for (int n = 9; n >= 0; --n) {
            s = s * w;
            s = s + ERF_SERIES[n];
        }
        return s * x;
    }
    float p = AS_7128[5];
    for (int i = 4; i >= 0; --i) {
        p = p * y;
        p = p + AS_7128[i];
    }
    p = p * y;
    p = p + 1.0f;
    float q = p * p;
    q = q * q;
    q = q * q;
    q = q * q;
    const float r = 1.0f / q;
    const float e = 1.0f - r;
    return copysignf(e, x);
}

/* GeLU(x) = x * Phi(x) = (x / 2) * (1 + erf(x / sqrt 2)), evaluated as
 * u = x * c with c = 1/sqrt(2) rounded to binary32; h = x * 0.5;
 * t = 1 + erf(u); GeLU = h * t. */
static float gelu_erf(float x)
{
    const float c = 0.70710678118654752440f;
    const float u = x * c;
    const float e = erf_piecewise(u);
    const float h = x * 0.5f;
    const float t = 1.0f + e;
    return h * t;
}

int repops_oracle_erf_f32(const float *x, float *y, int64_t n)
{
    if (n < 0) return -1;
    if (repops_oracle_env_status() != 0) return -2;
    for (int64_t i = 0; i < n; ++i) y[i] = erf_piecewise(x[i]);
    return 0;
}

int repops_oracle_gelu_f32(const float *x, float *y, int64_t n)
{
    if (n < 0) return -1;
    if (repops_oracle_env_status() != 0) return -2;
    for (int64_t i = 0; i < n; ++i) y[i] = gelu_erf(x[i]);
    return 0;
}

/* LayerNorm over each row of H elements (Ba, Kiros and Hinton, "Layer
 * Normalization", 2016: normalise by the mean and the biased variance of the
 * row, then scale by gamma and shift by beta).  Fixed order, per row r:
 *     S  = +0; for i ascending: S = S + x_i           mu  = S / H
 *     S2 = +0; for i ascending: d = x_i - mu; S2 = S2 + d*d
 *     var = S2 / H;  sd = sqrt(var + eps);  rstd = 1 / sd
 *     y_i = ((x_i - mu) * rstd) * gamma_i + beta_i
 * every operation rounded on its own (H <= 2^24 converts exactly).  gamma
 * and beta may be NULL (the multiply or the add is then left out).  mean and
 * rstd, when not NULL, receive mu and rstd per row.  Row r of x starts at
 * x + r * x_rs, of y at y + r * y_rs. */
int repops_oracle_layernorm_f32(const float *x, int64_t x_rs, const float *gamma,
                                const float *beta, float *y, int64_t y_rs, int64_t rows,
                                int64_t H, float eps, float *mean, float *rstd)
{
    if (rows < 0 || H < 1 || H > ((int64_t)1 << 24)) return -1;
    if (repops_oracle_env_status() != 0) return -2;
    const float fh = (float)H;
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = x + r * x_rs;
        float *yr = y + r * y_rs;
        float s = 0.0f;
        for (int64_t i = 0; i < H; ++i) s = s + xr[i];
        const float mu = s / fh;
        float s2 = 0.0f;
        for (int64_t i = 0; i < H; ++i) {
            const float d = xr[i] - mu;
            const float sq = d * d;
            s2 = s2 + sq;
        }
        const float var = s2 / fh;
        const float ve = var + eps;
        const float sd = sqrtf(ve);
        const float rs = 1.0f / sd;
        for (int64_t i = 0; i < H; ++i) {
            const float d = xr[i] - mu;
            float t = d * rs;
            if (gamma) t = t * gamma[i];
            if (beta) t = t + beta[i];
            yr[i] = t;
        }
        if (mean) mean[r] = mu;
        if (rstd) rstd[r] = rs;
    }
    return 0;
}
