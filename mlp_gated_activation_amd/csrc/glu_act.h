// glu_act.h -- device-side activation math shared by the elementwise, tiled
// and GEMM-epilogue kernels: the activations, their derivatives and the
// helpers they use.
//
// Sources (page title -- section):
//   [SWIGLU] "Write a Triton SiLU-Mul (SwiGLU) Kernel"
//   [LIGER]  "Kernel Profile: SwiGLU (Tier 1 -- Element-wise)"
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "glu_erfc.h"
#include "glu_internal.h"   // GLU_SCALED_EXP
#include "glu_taylor.h"

namespace glu {
namespace {

enum Kind { SILU = 0, GELU_ERF = 1, GELU_TANH = 2, RELU = 3 };

// ---------------------------------------------------------------------------
// Activations.  All sigmoids use e = exp(-|x|) so nothing overflows
// ([SWIGLU] "Kernel design rules": stable sigmoid for very negative x):
//   q = 1/(1+e);  sigmoid(x) = q (x >= 0) or e*q (x < 0).
// Derivatives are arranged so the one cancellation left (near act''s
// negative root) is a single well-conditioned sum.
// ---------------------------------------------------------------------------
__device__ inline float recip(float x) { return __builtin_amdgcn_rcpf(x); }   // x >= 1
__device__ inline float fabs_(float x) { return __builtin_fabsf(x); }
__device__ inline double fabs_(double x) { return __builtin_fabs(x); }
__device__ inline float fma_(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ inline double fma_(double a, double b, double c) { return __builtin_fma(a, b, c); }

// exp for the fp32 math of bf16/fp16 data: 2^(x log2 e) on the hardware
// exponential (exp2f keeps subnormal results).  Rounding x*log2(e) to fp32
// costs a relative error of about |x| * 6e-8 (under 4e-6 wherever a bf16 or
// fp16 result is not zero), far inside half an output ulp (2^-9 / 2^-12).
// Sigmoid pieces from a = |x| (or |w|) >= 0:  e = exp(-a), q = 1/(1 + e).
// fp32 (bf16/fp16 data): es = e * 2^16 = 2^(16 - a log2(e)) from the raw
// hardware exponential; es is normal for a < 98.4, and beyond that every
// product with e is below half the smallest bf16/fp16 subnormal, so the
// hardware's flush to zero there is harmless.  Rounding the argument near 16
// costs at most 6.6e-7 relative in e.  fp64 (fp32 data): see below.
struct SigParts {
    float e, q;
};
template <bool PRECISE = true> __device__ inline SigParts sig_parts(float a)
{
#if GLU_SCALED_EXP
    const float es = __builtin_amdgcn_exp2f(__builtin_fmaf(a, -1.44269504088896341f, 16.0f));
    return SigParts{es * 0x1p-16f, __builtin_amdgcn_rcpf(__builtin_fmaf(es, 0x1p-16f, 1.0f))};
#else
    const float e = exp2f(a * -1.44269504088896341f);
    return SigParts{e, __builtin_amdgcn_rcpf(1.0f + e)};
#endif
}
// fp64 (fp32 data).  exp(-a) = 2^k * exp(r), k = rint(-a log2 e), with
// r = -a - k ln2 reduced in two steps (ln2 = L1 + L2, L1 with 32 significant
// bits, so k * L1 is exact for the |k| <= 1587 here and the first step is an
// exact difference), |r| <= ln2/2 + 2^-40; exp(r) by its Taylor polynomial.
// This is Cody and Waite's additive argument reduction (W. J. Cody and
// W. Waite, "Software Manual for the Elementary Functions", 1980).  L1 is ln2
// truncated to 32 significant bits and L2 = ln2 - L1 rounded to fp64: the
// same two words as the ln2_hi / ln2_lo split of Sun's fdlibm exp (e_exp.c);
// tests/test_act_tables.py derives both from a 200-bit ln2.
// PRECISE (the backward): degree 12, truncation below |r|^13/13! * e^|r| <
// 3e-16 relative, so e carries a few fp64 ulps of error like a library exp,
// and the sums that cancel near act''s root, (1 + e) + x and its tanh form,
// stay as accurate as in exact arithmetic to within fp32 rounding.
// Otherwise (the forwards, whose products do not cancel): degree 7, below
// |r|^8/8! * e^|r| < 8e-9 relative, far inside fp32's 2^-24.
// a >= 0 is clamped to 1100, where exp(-a) is already 0 in fp64; NaN also
// goes to the clamp, so callers keep NaN through their product with x.
template <bool PRECISE> __device__ inline double exp_neg(double a)
{
    constexpr double kLog2eD = 1.4426950408889634074;
    constexpr double kLn2Hi = 6.93147180369123816490e-01, kLn2Lo = 1.90821492927058770002e-10;
    const double ac = a < 1100.0 ? a : 1100.0;
    const double k = __builtin_rint(ac * -kLog2eD);
    double r = __builtin_fma(k, -kLn2Hi, -ac);
    r = __builtin_fma(k, -kLn2Lo, r);
    constexpr double c[13] = {1.0, 1.0, 1.0 / 2, 1.0 / 6, 1.0 / 24, 1.0 / 120, 1.0 / 720, 1.0 / 5040,
                              1.0 / 40320, 1.0 / 362880, 1.0 / 3628800, 1.0 / 39916800, 1.0 / 479001600};
    constexpr int deg = PRECISE ? 12 : 7;
    double p = c[deg];
#pragma unroll
    for (int i = deg - 1; i >= 0; --i)
        p = __builtin_fma(p, r, c[i]);
    return __builtin_ldexp(p, int(k));
}
// 1/d for d >= 1: the hardware reciprocal, then Newton steps, each of which
// squares the relative error.  The seed measured within 4.6e-8 (2^-24.4)
// relative over d in [1, 128) on MI355X (2^24 points against the correctly
// rounded quotient); the arguments here stay in [1, 24].  One step (the
// forwards) leaves about 2^-48, two (PRECISE, the backward) fp64 rounding.
template <bool PRECISE = true> __device__ inline double recip_ge1(double d)
{
    double q = __builtin_amdgcn_rcp(d);
    q = __builtin_fma(q, __builtin_fma(-d, q, 1.0), q);
    if constexpr (PRECISE)
        q = __builtin_fma(q, __builtin_fma(-d, q, 1.0), q);
    return q;
}
struct SigPartsD {
    double e, q;
};
template <bool PRECISE = true> __device__ inline SigPartsD sig_parts(double a)
{
    const double e = exp_neg<PRECISE>(a);
    return SigPartsD{e, recip_ge1<PRECISE>(1.0 + e)};
}

constexpr double kInvSqrt2 = 0.70710678118654752440;      // [SWIGLU] reasoning step 7
constexpr double kInvSqrt2Pi = 0.39894228040143267794;
constexpr double kSqrt2OverPi = 0.79788456080286535588;   // [SWIGLU] failure modes
constexpr double kTanhCubic = 0.044715;

// Normal CDF Phi(x) and the density phi(x) in fp32, branch-free (see gen_erfc.py):
//   t = 1/(1 + |x|/(2 sqrt 2)),  h = Phi(-|x|) = 0.5 t Q(t) E,  E = exp(-x^2/2),
//   Phi = x >= 0 ? 1 - h : h,    phi = E / sqrt(2 pi).
// E is taken from the hardware exponential as Es = E * 2^16 = 2^(16 - x^2 log2(e)/2),
// which stays normal for |x| < 14 (beyond that Phi(-|x|) and phi are below
// every bf16/fp16 subnormal); the 2^-16 goes into the final products, which
// round subnormal results correctly.  One exp serves Phi and phi; no 1 + erf
// cancellation.  PRECISE (the backward, whose Phi + x phi cancels near its
// root): Q to 5.6e-7 relative, Phi about 1e-6 over all fp16/bf16 inputs.
// Otherwise (the forward x Phi(x)): the degree-5 table, Q to 6.5e-5, i.e.
// at most about 0.13 fp16 ulp of the result before its rounding.
constexpr float kLog2e = 1.44269504088896341f;
// norm_tail returns h = Phi(-|x|) and Es; norm_cdf turns them into Phi, phi.
template <bool PRECISE> __device__ inline float norm_tail(float x, float &Es)
{
    constexpr int deg = PRECISE ? GLU_ERFC_Q_DEG : GLU_ERFC_QF_DEG;
    constexpr float cp[GLU_ERFC_Q_DEG + 1] = GLU_ERFC_Q_COEFFS;
    constexpr float cf[GLU_ERFC_QF_DEG + 1] = GLU_ERFC_QF_COEFFS;
    const float t = recip(1.0f + fabs_(x) * float(0.5 * kInvSqrt2));
    // Q's coefficients carry the 2^-17 that undoes the exponent offset below:
    // scaling by a power of two commutes with every rounding here (all values
    // stay normal), so this equals scaling t*Q afterwards, one multiply less.
    constexpr float kS = 0x1p-17f;
    float q = (PRECISE ? cp[deg] : cf[deg]) * kS;
#pragma unroll
    for (int k = deg - 1; k >= 0; --k)
        q = fma_(q, t, (PRECISE ? cp[k] : cf[k]) * kS);
    Es = __builtin_amdgcn_exp2f(fma_(x * x, -0.5f * kLog2e, 16.0f));
    return (t * q) * Es;
}
template <bool PRECISE = true> __device__ inline void norm_cdf(float x, float &Phi, float &phi)
{
    float Es;
    const float h = norm_tail<PRECISE>(x, Es);
    Phi = x >= 0.0f ? 1.0f - h : h;
    phi = Es * float(kInvSqrt2Pi * 0x1p-16);
}
// x * Phi(x) = relu(x) - |x| h for either sign (Phi = 1 - h for x >= 0, h
// below): one fma, so one rounding instead of two, and no select.  |x| is
// clamped to 64, past which h is 0, so +inf gives +inf rather than inf * 0;
// NaN stays NaN through h.
__device__ inline float x_phi(float x, float h)
{
    return fma_(-__builtin_fminf(fabs_(x), 64.0f), h, __builtin_fmaxf(x, 0.0f));
}
__device__ inline double x_phi(double x, double h)
{
    return fma_(-__builtin_fmin(fabs_(x), 64.0), h, __builtin_fmax(x, 0.0));
}

// Phi(x) and phi(x) in fp64 for fp32 data, by the same substitution as
// norm_cdf with fp64 tables, exp_neg and the reciprocal above.  PRECISE (the
// backward): Q to 4.6e-10 relative, so Phi within about 5e-10 and phi within
// a few fp64 ulps.  Otherwise (the forward): Q to 1.7e-7 and the shorter exp
// and reciprocal, Phi(-|x|) within about 1.8e-7.  The forward x * Phi(x)
// carries that relative error (for x >= 0, x - |x| h with h <= 1/2 at most
// doubles an absolute error of h that is itself at most half its relative
// one), so with its one rounding to fp32 it stays below 2.5e-7, a quarter of
// the 1e-6 bound; the backward's Phi + x phi
// cancels near its root, where a Taylor expansion in fp64 takes over
// (taylor_patch_d).  |x| is clamped to 64, beyond which Phi(-|x|) and phi
// are 0 in fp64; NaN passes the clamp and makes h NaN.
template <bool PRECISE> __device__ inline double norm_tail_d(double x, double &E)
{
    constexpr int deg = PRECISE ? GLU_ERFC_QD_DEG : GLU_ERFC_QDF_DEG;
    constexpr double cp[GLU_ERFC_QD_DEG + 1] = GLU_ERFC_QD_COEFFS;
    constexpr double cf[GLU_ERFC_QDF_DEG + 1] = GLU_ERFC_QDF_COEFFS;
    const double ax = fabs_(x) > 64.0 ? 64.0 : fabs_(x);
    const double t = recip_ge1<PRECISE>(__builtin_fma(ax, 0.5 * kInvSqrt2, 1.0));
    double q = PRECISE ? cp[deg] : cf[deg];
#pragma unroll
    for (int k = deg - 1; k >= 0; --k)
        q = __builtin_fma(q, t, PRECISE ? cp[k] : cf[k]);
    E = exp_neg<PRECISE>(0.5 * ax * ax);
    return 0.5 * t * q * E;
}
template <bool PRECISE> __device__ inline void norm_cdf_d(double x, double &Phi, double &phi)
{
    double E;
    const double h = norm_tail_d<PRECISE>(x, E);
    Phi = x >= 0.0 ? 1.0 - h : h;
    phi = E * kInvSqrt2Pi;
}

// GELU-erf's derivative near its root for fp32 data (fp64; see gen_taylor.py):
// inside |x - x0| < 1/32 the expansion, good to 1.5e-13 relative, replaces
// Phi + x phi, whose table error (5e-10 of Phi ~ 0.23) would otherwise be
// magnified by the cancellation; outside, that error stays below 1e-8
// relative.
__device__ inline double taylor_patch_d(double x, double d)
{
    constexpr double c[GLU_TAYLOR_GELU_ERF_D_DEG] = GLU_TAYLOR_GELU_ERF_D_COEFFS;
    const double h = x - GLU_TAYLOR_GELU_ERF_D_X0_HI;   // exact inside the zone
    const double t = h - GLU_TAYLOR_GELU_ERF_D_X0_LO;
    double p = c[GLU_TAYLOR_GELU_ERF_D_DEG - 1];
#pragma unroll
    for (int k = GLU_TAYLOR_GELU_ERF_D_DEG - 2; k >= 0; --k)
        p = __builtin_fma(p, t, c[k]);
    return __builtin_fabs(h) < 1.0 / 32.0 ? p * t : d;
}

// Clamp for the tanh form's polynomial: beyond |x| = 16 its sigmoid is 0 or
// 1 in fp32 (and its contribution below any fp32/bf16/fp16 subnormal), while
// x^3 would overflow.  NaN passes through.
template <typename M> __device__ inline M tanh_clamp(M x)
{
    return x > M(16) ? M(16) : (x < M(-16) ? M(-16) : x);
}

template <int KIND, typename M> __device__ inline M act(M x)
{
    if constexpr (KIND == SILU) {
        // silu(x) = x * sigmoid(x): [SWIGLU] reasoning step 5; [LIGER] Forward Pass
        const auto sp = sig_parts<false>(fabs_(x));
        return x * (sp.q * (x >= M(0) ? M(1) : sp.e));
    } else if constexpr (KIND == GELU_ERF) {
        // x * Phi(x), Phi(x) = (1 + erf(x/sqrt2))/2 = erfc(-x/sqrt2)/2: reasoning step 7
        M E;
        if constexpr (sizeof(M) == 4)
            return x_phi(x, norm_tail<false>(x, E));
        else
            return x_phi(x, norm_tail_d<false>(x, E));
    } else if constexpr (KIND == GELU_TANH) {
        // 0.5*x*(1+tanh(u)) = x * sigmoid(2u), u = sqrt(2/pi)(x + 0.044715 x^3)
        M xc = tanh_clamp(x);
        M w = xc * fma_(M(2 * kSqrt2OverPi * kTanhCubic), xc * xc, M(2 * kSqrt2OverPi));
        const auto sp = sig_parts<false>(fabs_(w));
        return x * (sp.q * (w >= M(0) ? M(1) : sp.e));
    } else {
        // relu, NaN-propagating: [SWIGLU] Purpose (ReGLU)
        return x > M(0) ? x : (x != x ? x : M(0));
    }
}

// Polynomial for act' near its root (fp16 only; see gen_taylor.py).
template <int KIND> __device__ inline float taylor_patch(float x, float d)
{
    constexpr float R = GLU_TAYLOR_RADIUS;
    float hi, lo;
    float c[4];
    if constexpr (KIND == SILU) {
        hi = GLU_TAYLOR_SILU_X0_HI; lo = GLU_TAYLOR_SILU_X0_LO;
        const float cc[GLU_TAYLOR_SILU_DEG] = GLU_TAYLOR_SILU_COEFFS;
        for (int k = 0; k < 4; ++k) c[k] = cc[k];
    } else if constexpr (KIND == GELU_ERF) {
        hi = GLU_TAYLOR_GELU_ERF_X0_HI; lo = GLU_TAYLOR_GELU_ERF_X0_LO;
        const float cc[GLU_TAYLOR_GELU_ERF_DEG] = GLU_TAYLOR_GELU_ERF_COEFFS;
        for (int k = 0; k < 4; ++k) c[k] = cc[k];
    } else {
        hi = GLU_TAYLOR_GELU_TANH_X0_HI; lo = GLU_TAYLOR_GELU_TANH_X0_LO;
        const float cc[GLU_TAYLOR_GELU_TANH_DEG] = GLU_TAYLOR_GELU_TANH_COEFFS;
        for (int k = 0; k < 4; ++k) c[k] = cc[k];
    }
    float h = x - hi;                  // exact (Sterbenz) inside the zone
    float t = h - lo;
    float p = __builtin_fmaf(c[3], t, c[2]);
    p = __builtin_fmaf(p, t, c[1]);
    p = __builtin_fmaf(p, t, c[0]);
    return __builtin_fabsf(h) < R ? p * t : d;
}

// f = act(x) and g = act'(x) together (backward).
template <int KIND, bool PATCH, typename M> __device__ inline void act_grad(M x, M &f, M &g)
{
    if constexpr (KIND == SILU) {
        // silu' = s*(1 + x*(1-s)): [SWIGLU] correctness requirements; [LIGER]
        // Backward Pass.  With e = exp(-|x|), q = 1/(1+e):
        //   x >= 0:  q^2 * ((1+e) + x*e)
        //   x <  0:  e*q^2 * ((1+e) + x)     (the root's cancellation is this one sum)
        // i.e. g = q^2 * s * fma(x, m, 1+e) with (s, m) = (1, e) or (e, 1):
        // selects only, no divergent branch.
        const auto sp = sig_parts(fabs_(x));
        const M e = sp.e, q = sp.q;
        bool pos = x >= M(0);
        M sg = pos ? M(1) : e;
        M m = pos ? e : M(1);
        f = x * (q * sg);
        g = (q * q) * sg * fma_(x, m, M(1) + e);
    } else if constexpr (KIND == GELU_ERF) {
        // d/dx [x Phi(x)] = Phi(x) + x phi(x)
        M Phi, phi;
        if constexpr (sizeof(M) == 4)
            norm_cdf(x, Phi, phi);
        else
            norm_cdf_d<true>(x, Phi, phi);
        f = x * Phi;
        g = fma_(x, phi, Phi);
        if constexpr (sizeof(M) == 8)
            g = taylor_patch_d(x, g);
    } else if constexpr (KIND == GELU_TANH) {
        // w = 2u, v = 2x u'; sigmoid(w) (1 + v sigmoid(-w)):
        //   w >= 0:  q^2 * ((1+e) + v*e)
        //   w <  0:  e*q^2 * ((1+e) + v)
        // folded into selects as for silu'.
        M xc = tanh_clamp(x);
        M x2 = xc * xc;
        M w = xc * fma_(M(2 * kSqrt2OverPi * kTanhCubic), x2, M(2 * kSqrt2OverPi));
        M v = xc * fma_(M(6 * kSqrt2OverPi * kTanhCubic), x2, M(2 * kSqrt2OverPi));
        const auto sp = sig_parts(fabs_(w));
        const M e = sp.e, q = sp.q;
        bool pos = w >= M(0);
        M sg = pos ? M(1) : e;
        M m = pos ? e : M(1);
        f = x * (q * sg);
        g = (q * q) * sg * fma_(v, m, M(1) + e);
        if (x != x)
            g = x;
    } else {
        f = x > M(0) ? x : (x != x ? x : M(0));
        g = x > M(0) ? M(1) : (x != x ? x : M(0));
    }
    if constexpr (PATCH && KIND != RELU)
        g = taylor_patch<KIND>(x, g);
}

}  // namespace
}  // namespace glu
