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
__device__ inline float recip(float x) { return __builtin_amdgcn_rcpf(x); }   // x in [1, 2]
__device__ inline double recip(double x) { return 1.0 / x; }
__device__ inline float fabs_(float x) { return __builtin_fabsf(x); }
__device__ inline double fabs_(double x) { return __builtin_fabs(x); }
__device__ inline float fma_(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ inline double fma_(double a, double b, double c) { return __builtin_fma(a, b, c); }

// exp for the fp32 math of bf16/fp16 data: 2^(x log2 e) on the hardware
// exponential (exp2f keeps subnormal results).  Rounding x*log2(e) to fp32
// costs a relative error of about |x| * 6e-8 (under 4e-6 wherever a bf16 or
// fp16 result is not zero), far inside half an output ulp (2^-9 / 2^-12).
// The fp64 math of fp32 data uses the library exp.
// Sigmoid pieces from a = |x| (or |w|) >= 0:  e = exp(-a), q = 1/(1 + e).
// fp32 (bf16/fp16 data): es = e * 2^16 = 2^(16 - a log2(e)) from the raw
// hardware exponential; es is normal for a < 98.4, and beyond that every
// product with e is below half the smallest bf16/fp16 subnormal, so the
// hardware's flush to zero there is harmless.  Rounding the argument near 16
// costs at most 6.6e-7 relative in e.  fp64 (fp32 data): library exp.
struct SigParts {
    float e, q;
};
__device__ inline SigParts sig_parts(float a)
{
#if GLU_SCALED_EXP
    const float es = __builtin_amdgcn_exp2f(__builtin_fmaf(a, -1.44269504088896341f, 16.0f));
    return SigParts{es * 0x1p-16f, __builtin_amdgcn_rcpf(__builtin_fmaf(es, 0x1p-16f, 1.0f))};
#else
    const float e = exp2f(a * -1.44269504088896341f);
    return SigParts{e, __builtin_amdgcn_rcpf(1.0f + e)};
#endif
}
struct SigPartsD {
    double e, q;
};
__device__ inline SigPartsD sig_parts(double a)
{
    const double e = exp(-a);
    return SigPartsD{e, 1.0 / (1.0 + e)};
}

template <typename M> __device__ inline M ex(M x);
template <> __device__ inline float ex<float>(float x) { return exp2f(x * 1.44269504088896341f); }
template <> __device__ inline double ex<double>(double x) { return exp(x); }
template <typename M> __device__ inline M erfc_(M x);
template <> __device__ inline float erfc_<float>(float x) { return erfcf(x); }
template <> __device__ inline double erfc_<double>(double x) { return erfc(x); }

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
template <bool PRECISE = true> __device__ inline void norm_cdf(float x, float &Phi, float &phi)
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
    const float Es = __builtin_amdgcn_exp2f(fma_(x * x, -0.5f * kLog2e, 16.0f));
    const float h = (t * q) * Es;
    Phi = x >= 0.0f ? 1.0f - h : h;
    phi = Es * float(kInvSqrt2Pi * 0x1p-16);
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
        const auto sp = sig_parts(fabs_(x));
        return x * (sp.q * (x >= M(0) ? M(1) : sp.e));
    } else if constexpr (KIND == GELU_ERF) {
        // x * Phi(x), Phi(x) = (1 + erf(x/sqrt2))/2 = erfc(-x/sqrt2)/2: reasoning step 7
        if constexpr (sizeof(M) == 4) {
            float Phi, phi;
            norm_cdf<false>(x, Phi, phi);
            return x * Phi;
        } else {
            return x * (M(0.5) * erfc_<M>(x * M(-kInvSqrt2)));
        }
    } else if constexpr (KIND == GELU_TANH) {
        // 0.5*x*(1+tanh(u)) = x * sigmoid(2u), u = sqrt(2/pi)(x + 0.044715 x^3)
        M xc = tanh_clamp(x);
        M w = xc * fma_(M(2 * kSqrt2OverPi * kTanhCubic), xc * xc, M(2 * kSqrt2OverPi));
        const auto sp = sig_parts(fabs_(w));
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
        if constexpr (sizeof(M) == 4) {
            norm_cdf(x, Phi, phi);
        } else {
            Phi = M(0.5) * erfc_<M>(x * M(-kInvSqrt2));
            phi = ex<M>(M(-0.5) * x * x) * M(kInvSqrt2Pi);
        }
        f = x * Phi;
        g = fma_(x, phi, Phi);
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
