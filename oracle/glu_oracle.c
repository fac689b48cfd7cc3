/*
 * glu_oracle.c -- fp64 scalar reference for the fused gated activation
 *                 y = act(a) * b and its backward.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the HIP path is
 * checked against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, constant or helper
 * with the GPU library, and the GPU library never calls it.
 *
 * Every function is the plain mathematical definition, evaluated in IEEE
 * double precision with the host C library (exp, erfc), one element at a
 * time, with no final rounding: callers compare the GPU's stored result
 * against the unrounded double value.  OpenMP only splits the element loop
 * across threads; each element's arithmetic is independent of the split.
 *
 * Sources (page title -- section):
 *  [SWIGLU]  "Write a Triton SiLU-Mul (SwiGLU) Kernel"
 *  [LIGER]   "Kernel Profile: SwiGLU (Tier 1 -- Element-wise)" (Liger-Kernel)
 *  [FUSED]   "Fused Kernels" (lesson 5)
 *  [RMSNORM] "Write a Triton Fused Add+RMSNorm Kernel"
 *  [FUSED]   "Fused Kernels" (lesson 5), section 4 (the fused MLP)
 *
 * Readings where the pages leave a step open (all pinned by tests):
 *  - GELU-erf is evaluated as 0.5*x*erfc(-x/sqrt2), which equals the pages'
 *    0.5*x*(1+erf(x/sqrt2)) but does not cancel to zero for x << 0.
 *  - GELU-tanh's 0.5*(1+tanh(u)) is evaluated as sigmoid(2u) (an identity),
 *    for the same reason.
 *  - The GeGLU and ReGLU derivatives are not printed on the pages; they are
 *    the derivatives of the forward definitions.  relu'(0) = 0.
 *  - NaN inputs propagate to NaN outputs for every kind (ReLU included).
 */
#include <math.h>
#include <stdint.h>

#define ORACLE_SILU 0
#define ORACLE_GELU_ERF 1
#define ORACLE_GELU_TANH 2
#define ORACLE_RELU 3

/* 1/sqrt(2): the constant [SWIGLU] "Required reasoning process", step 7 prints. */
static const double INV_SQRT2 = 0.70710678118654752440;
/* 1/sqrt(2*pi), the normal density's constant. */
static const double INV_SQRT_2PI = 0.39894228040143267794;
/* sqrt(2/pi) and 0.044715: [SWIGLU] "Common failure modes", GELU variant mismatch. */
static const double SQRT_2_OVER_PI = 0.79788456080286535588;
static const double GELU_TANH_C = 0.044715;

/* Logistic sigmoid, in the form that never overflows exp():
 * [SWIGLU] "Kernel design rules" asks for a sigmoid that is stable for very
 * negative x. */
static double sigmoid(double x)
{
    if (x >= 0.0)
        return 1.0 / (1.0 + exp(-x));
    double e = exp(x);
    return e / (1.0 + e);
}

/* silu(x) = x * sigmoid(x): [SWIGLU] "Purpose" and "Inputs", item 1;
 * [LIGER] "Forward Pass". */
static double silu(double x) { return x * sigmoid(x); }

/* Standard normal CDF Phi(x) = 0.5*(1+erf(x/sqrt2)) = 0.5*erfc(-x/sqrt2). */
static double phi_cdf(double x) { return 0.5 * erfc(-x * INV_SQRT2); }

/* Standard normal density. */
static double phi_pdf(double x) { return INV_SQRT_2PI * exp(-0.5 * x * x); }

/* GELU, erf form: x * Phi(x).  [SWIGLU] "Inputs", item 2, and
 * "Required reasoning process", step 7. */
static double gelu_erf(double x) { return x * phi_cdf(x); }

/* tanh-approximation GELU: 0.5*x*(1+tanh(k*(x+0.044715*x^3))), k=sqrt(2/pi).
 * [SWIGLU] "Common failure modes", GELU variant mismatch. */
static double gelu_tanh_u(double x) { return SQRT_2_OVER_PI * (x + GELU_TANH_C * x * x * x); }
static double gelu_tanh(double x) { return x * sigmoid(2.0 * gelu_tanh_u(x)); }

/* relu(x) = max(x, 0): [SWIGLU] "Purpose" (ReGLU). */
static double relu(double x)
{
    if (isnan(x))
        return x;
    return x > 0.0 ? x : 0.0;
}

/* silu'(x) = sigmoid(x) * (1 + x*(1 - sigmoid(x))):
 * [SWIGLU] "Correctness requirements" (last item); [LIGER] "Backward Pass"
 * gives the equal form silu(x)*(1-sigmoid(x)) + sigmoid(x). */
static double dsilu(double x)
{
    double s = sigmoid(x);
    return s * (1.0 + x * (1.0 - s));
}

/* d/dx [x*Phi(x)] = Phi(x) + x*phi(x).  Derived from the erf-form forward. */
static double dgelu_erf(double x) { return phi_cdf(x) + x * phi_pdf(x); }

/* d/dx [0.5*x*(1+tanh(u))] = 0.5*(1+tanh(u)) + 0.5*x*(1-tanh(u)^2)*u',
 * u' = k*(1+3*0.044715*x^2).  With 0.5*(1+tanh(u)) = sigmoid(2u) and
 * 1-tanh(u)^2 = 4*sigmoid(2u)*sigmoid(-2u).  Derived from the tanh forward. */
static double dgelu_tanh(double x)
{
    double u = gelu_tanh_u(x);
    double du = SQRT_2_OVER_PI * (1.0 + 3.0 * GELU_TANH_C * x * x);
    double sp = sigmoid(2.0 * u);
    double sm = sigmoid(-2.0 * u);
    return sp + 2.0 * x * du * sp * sm;
}

/* relu'(x) = 1 for x > 0, else 0 (0 at x == 0).  Derived. */
static double drelu(double x)
{
    if (isnan(x))
        return x;
    return x > 0.0 ? 1.0 : 0.0;
}

double oracle_act(int kind, double x)
{
    switch (kind) {
    case ORACLE_SILU: return silu(x);
    case ORACLE_GELU_ERF: return gelu_erf(x);
    case ORACLE_GELU_TANH: return gelu_tanh(x);
    case ORACLE_RELU: return relu(x);
    default: return NAN;
    }
}

double oracle_dact(int kind, double x)
{
    switch (kind) {
    case ORACLE_SILU: return dsilu(x);
    case ORACLE_GELU_ERF: return dgelu_erf(x);
    case ORACLE_GELU_TANH: return dgelu_tanh(x);
    case ORACLE_RELU: return drelu(x);
    default: return NAN;
    }
}

/* Elementwise act / act' over n values (used by the pins). */
void oracle_act_n(int kind, int64_t n, const double *x, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_act(kind, x[i]);
}

void oracle_dact_n(int kind, int64_t n, const double *x, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_dact(kind, x[i]);
}

/* Forward: y = act(a) * b, elementwise over n values.
 * [SWIGLU] "Required reasoning process", steps 5-7; [LIGER] "Forward Pass";
 * [FUSED] section 3 (the silu gate). */
void oracle_fwd(int kind, int64_t n, const double *a, const double *b, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        y[i] = oracle_act(kind, a[i]) * b[i];
}

/* Backward: da = dy * act'(a) * b,  db = dy * act(a), elementwise.
 * [SWIGLU] "Required reasoning process", step 9; [LIGER] "Backward Pass"
 * (gradient formulas, recomputing sigmoid from the saved a). */
void oracle_bwd(int kind, int64_t n, const double *a, const double *b, const double *dy,
                double *da, double *db)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double x = a[i];
        da[i] = dy[i] * oracle_dact(kind, x) * b[i];
        db[i] = dy[i] * oracle_act(kind, x);
    }
}

/* Fused residual add + RMSNorm forward, one row of H values at a time
 * ([RMSNORM] "Required reasoning process", steps 1-7, and "Correctness
 * requirements"):
 *   h = x + residual,  rstd = 1 / sqrt(sum_j h_j^2 / H + eps),
 *   y = h * rstd * gamma_j   (gamma indexed by column only),
 * with the mean over all H columns, eps inside the square root, no mean
 * subtraction and no bias.  h, y: rows*H values; rstd: rows values or NULL.
 * Statistics and y use the exact sum h (the reading of the single-pass form,
 * where h stays in fp32 registers), not h rounded to the storage dtype. */
void oracle_add_rmsnorm(int64_t rows, int64_t H, const double *x, const double *res,
                        const double *gamma, double eps, double *h, double *y, double *rstd)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        const double *xi = x + i * H, *ri = res + i * H;
        double *hi = h + i * H, *yi = y + i * H;
        double ss = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            hi[j] = xi[j] + ri[j];
            ss += hi[j] * hi[j];
        }
        double rs = 1.0 / sqrt(ss / (double)H + eps);
        for (int64_t j = 0; j < H; ++j)
            yi[j] = hi[j] * rs * gamma[j];
        if (rstd)
            rstd[i] = rs;
    }
}

/* Gate/up projection with the gated activation fused into it ([FUSED]
 * section 4: gate and up tiles are accumulated, then silu(g) * u is applied
 * in registers; [SWIGLU] "Do not use this when" and "Performance
 * requirements": the activation fused into the matmul epilogue):
 *   g[m][n] = sum_k x[m][k] * wg[n][k]
 *   u[m][n] = sum_k x[m][k] * wu[n][k]
 *   h[m][n] = act(g[m][n]) * u[m][n]
 * x is M x K, wg and wu are N x K (the [out][in] layout of a linear layer's
 * weight), all dense row-major.  The sums run over k in order in fp64
 * (products of 16-bit inputs are exact in fp64); nothing is rounded to a
 * storage type.  g and u may be NULL. */
void oracle_gemm_glu(int kind, int64_t M, int64_t N, int64_t K, const double *x, const double *wg,
                     const double *wu, double *h, double *g, double *u)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        const double *xm = x + m * K;
        for (int64_t n = 0; n < N; ++n) {
            const double *gn = wg + n * K, *un = wu + n * K;
            double sg = 0.0, su = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                sg += xm[k] * gn[k];
                su += xm[k] * un[k];
            }
            h[m * N + n] = oracle_act(kind, sg) * su;
            if (g)
                g[m * N + n] = sg;
            if (u)
                u[m * N + n] = su;
        }
    }
}

/* Thread count OpenMP will use for the loops above (1 without OpenMP), and
 * a way to change it (n >= 1) for single-thread timings. */
#ifdef _OPENMP
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
void oracle_set_num_threads(int n) { omp_set_num_threads(n < 1 ? 1 : n); }
#else
int oracle_num_threads(void) { return 1; }
void oracle_set_num_threads(int n) { (void)n; }
#endif
