/*
 * glu.h -- C ABI of the MI355X (gfx950) fused gated-activation library.
 *
 * Computes the activation step of a gated MLP between its gate/up and down
 * projections, y = act(a) * b, and its backward, for
 *   act = SiLU (SwiGLU), GELU erf form and GELU tanh form (GeGLU), ReLU (ReGLU).
 *
 * Sources (page title -- section):
 *   [SWIGLU] "Write a Triton SiLU-Mul (SwiGLU) Kernel"
 *   [LIGER]  "Kernel Profile: SwiGLU (Tier 1 -- Element-wise)"
 *   [FUSED]  "Fused Kernels"
 *
 * Conventions shared by every entry point:
 *  - A tensor is a row-major matrix of `rows` rows.  Row strides (`ld*`) are
 *    in ELEMENTS; the column stride is always 1 ([SWIGLU] "Inputs", item 3:
 *    the activation dimension is the last, contiguous one).
 *  - One dtype for every operand, inputs and outputs alike ([SWIGLU]
 *    "Inputs", item 6: the output usually keeps the input dtype).
 *  - bf16/fp16 data is computed in fp32 and rounded once, to nearest-even, at
 *    the store ([SWIGLU] "Kernel design rules"); fp32 data is computed in fp64
 *    and rounded once.  Results are within one unit in the last place of the
 *    output dtype of the exact value.
 *  - Pointers are DEVICE pointers owned by the caller.  The library never
 *    allocates, frees, caches or keeps them, has no global state, needs no
 *    workspace and is safe to call from several host threads.
 *  - Every call validates all arguments on the host before any HIP call; on
 *    error nothing is enqueued.  On success exactly one kernel launch per
 *    2^30 16-byte vectors is enqueued on `stream` (NULL = the null stream)
 *    and the call returns without synchronising; buffers must stay alive
 *    until the stream reaches that point.  Device faults surface at the
 *    caller's next synchronisation, as usual in HIP.
 *  - rows == 0 or cols == 0 is a successful no-op (pointers may then be NULL).
 *  - Alignment is never required.  When every pointer, row stride and half
 *    offset is a multiple of 16 bytes the kernels move 16-byte vectors;
 *    otherwise they fall back to per-element access.
 *  - An output may coincide EXACTLY with an input (same pointer, same row
 *    stride): each element is read by the lane that later writes it, before
 *    it writes it ([SWIGLU] "Common failure modes", in-place store).  Any
 *    other overlap of an output with an input, or of two outputs, is
 *    rejected with GLU_ERR_ALIAS.
 */
#ifndef GLU_H
#define GLU_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exported entry points (the library is built with hidden visibility). */
#ifndef GLU_API
#define GLU_API __attribute__((visibility("default")))
#endif

/* The activation.  [SWIGLU] "Inputs", items 1-2; "Common failure modes"
 * (the tanh form is 0.5*x*(1+tanh(sqrt(2/pi)*(x+0.044715*x^3))), not
 * interchangeable with the erf form 0.5*x*(1+erf(x/sqrt2))). */
typedef enum {
    GLU_SILU = 0,      /* silu(x) = x * sigmoid(x)            (SwiGLU) */
    GLU_GELU_ERF = 1,  /* x * Phi(x), Phi the normal CDF       (GeGLU)  */
    GLU_GELU_TANH = 2, /* tanh approximation of GELU           (GeGLU)  */
    GLU_RELU = 3       /* max(x, 0); relu'(0) = 0              (ReGLU)  */
} glu_kind;

/* Where a and b live.  [SWIGLU] "Inputs", item 4, and "Correctness
 * requirements": a fused gate/up GEMM yields one (rows, 2*cols) tensor
 * whose first `cols` columns are the gate a (activated) and whose last
 * `cols` columns are the up projection b. */
typedef enum {
    GLU_SEPARATE = 0, /* a and b are two (rows, cols) matrices                */
    GLU_GATE_UP = 1   /* x = [a | b], (rows, 2*cols), a = x[:, :cols], b = x[:, cols:] */
} glu_layout;

typedef enum { GLU_F32 = 0, GLU_F16 = 1, GLU_BF16 = 2 } glu_dtype;

typedef enum {
    GLU_OK = 0,
    GLU_ERR_NULL = 1,    /* a required pointer is NULL, or a must-be-NULL one is not */
    GLU_ERR_SHAPE = 2,   /* rows < 0, cols < 0, or the extent overflows int64 bytes */
    GLU_ERR_STRIDE = 3,  /* a row stride below the row width (cols; 2*cols for x)   */
    GLU_ERR_ENUM = 4,    /* kind, layout or dtype out of range                      */
    GLU_ERR_ALIAS = 5,   /* an output overlaps an input other than exactly, or another output */
    GLU_ERR_INPLACE = 6, /* inplace not 0/1, or output pointers given with inplace = 1 */
    GLU_ERR_HIP = 7,     /* the kernel launch returned a HIP error                  */
    GLU_ERR_ARG = 8      /* a scalar argument out of range (eps must be finite and > 0), or a
                            strided operand's pointer not aligned to its element size */
} glu_status;

/*
 * Forward: y = act(a) * b, elementwise.
 * [SWIGLU] "Required reasoning process", steps 1-8; [LIGER] "Forward Pass";
 * [FUSED] section 3 (the silu gate).
 *
 *   SEPARATE: a (rows, cols, row stride lda) is the gate, b (rows, cols, ldb)
 *             the up projection.
 *   GATE_UP:  a points at x (rows, 2*cols, row stride lda >= 2*cols);
 *             b must be NULL and ldb is ignored.
 *   inplace = 0: y (rows, cols, ldy) receives the result.
 *   inplace = 1: y must be NULL; the result overwrites b, i.e. b itself
 *             (SEPARATE, with ldb) or the up half x[:, cols:] (GATE_UP, with
 *             lda) ([SWIGLU] "Inputs", item 7).
 * a and b are read-only except for that in-place write.
 */
GLU_API glu_status glu_fwd(glu_kind kind, glu_layout layout, glu_dtype dtype,
                   int64_t rows, int64_t cols,
                   void *a, int64_t lda,
                   void *b, int64_t ldb,
                   void *y, int64_t ldy,
                   int inplace, hipStream_t stream);

/*
 * Backward: da = dy * act'(a) * b,  db = dy * act(a), elementwise, with
 * sigmoid / Phi recomputed from a (nothing saved from the forward but a, b).
 * [SWIGLU] "Required reasoning process", step 9; [LIGER] "Backward Pass" and
 * "Key Patterns" (recompute, write the gradients over the saved a and b).
 * The GeGLU and ReGLU derivatives are those of their forward definitions.
 *
 *   SEPARATE: a (rows, cols, lda), b (rows, cols, ldb).
 *   GATE_UP:  a points at x (rows, 2*cols, lda >= 2*cols); b must be NULL.
 *   dy (rows, cols, lddy) is the incoming gradient of y.
 *   inplace = 1: da and db must be NULL; da overwrites a and db overwrites b
 *             (GATE_UP: dx = [da | db] overwrites x).
 *   inplace = 0: SEPARATE: da (rows, cols, ldda) and db (rows, cols, lddb).
 *             GATE_UP: da points at dx (rows, 2*cols, ldda >= 2*cols), which
 *             receives [da | db]; db must be NULL and lddb is ignored.
 * a, b and dy are read-only except for the in-place writes.
 */
GLU_API glu_status glu_bwd(glu_kind kind, glu_layout layout, glu_dtype dtype,
                   int64_t rows, int64_t cols,
                   void *a, int64_t lda,
                   void *b, int64_t ldb,
                   const void *dy, int64_t lddy,
                   void *da, int64_t ldda,
                   void *db, int64_t lddb,
                   int inplace, hipStream_t stream);

/*
 * The same forward and backward on operands of any 2-D layout: element
 * (r, c) of operand t lives at t + r*t_rs + c*t_cs (strides in ELEMENTS,
 * both >= 0; pointers aligned to the element size), so transposed, sliced
 * and broadcast (stride 0) views need no copy ("Write a Triton SiLU-Mul
 * (SwiGLU) Kernel", Kernel design rules and Common failure modes: strides
 * come from the tensor's metadata, and a transposed view must either be
 * made contiguous or have its strides threaded through the kernel).  The [gate | up] layout is the two views x and x + cols*cs.
 *
 * Outputs (y; da, db) must not map two (r, c) to one address
 * (GLU_ERR_STRIDE otherwise).  An output may coincide exactly with an input
 * (same pointer and both strides: the in-place forms); any other overlap of
 * an output with an input or with the other output is GLU_ERR_ALIAS.
 * When every operand is row-major (column stride 1) or every operand is
 * column-major (row stride 1) the 16-byte streaming kernels run; otherwise
 * 64 x 64 tiles are staged through LDS so each operand is still read or
 * written along its own contiguous direction.
 */
GLU_API glu_status glu_fwd_strided(glu_kind kind, glu_dtype dtype, int64_t rows, int64_t cols,
                           const void *a, int64_t a_rs, int64_t a_cs,
                           const void *b, int64_t b_rs, int64_t b_cs,
                           void *y, int64_t y_rs, int64_t y_cs,
                           hipStream_t stream);

GLU_API glu_status glu_bwd_strided(glu_kind kind, glu_dtype dtype, int64_t rows, int64_t cols,
                           const void *a, int64_t a_rs, int64_t a_cs,
                           const void *b, int64_t b_rs, int64_t b_cs,
                           const void *dy, int64_t dy_rs, int64_t dy_cs,
                           void *da, int64_t da_rs, int64_t da_cs,
                           void *db, int64_t db_rs, int64_t db_cs,
                           hipStream_t stream);

/*
 * Gate/up projection with the gated activation fused into its epilogue
 * ("Fused Kernels", section 4: the gate and up tiles are accumulated and
 * silu(g) * u is applied in registers; "Write a Triton SiLU-Mul (SwiGLU)
 * Kernel", Do not use this when and Performance requirements: fusing the
 * activation into the matmul epilogue saves the round trip of g and u
 * through HBM):
 *
 *   g[m][n] = sum_k x[m][k] * w_gate[n][k],  u[m][n] = sum_k x[m][k] * w_up[n][k],
 *   h[m][n] = act(g[m][n]) * u[m][n]
 *
 * x is M x K (row stride ldx), w_gate and w_up are N x K: the [out][in]
 * layout of a linear layer's weight (for one fused [gate | up] weight of
 * 2N rows, w_up = w_gate + N * ldw).  h is M x N (row stride ldh).  The
 * products accumulate in fp32 on the matrix cores; act(g) * u is evaluated
 * in fp32 and rounded once (RNE) to the storage type.
 * gu (optional, NULL to skip): the pre-activations, rounded to the storage
 * type, in the [gate | up] layout: g at gu[m][n], u at gu[m][N + n], row
 * stride ldgu >= 2N.  That is the input glu_bwd takes with GLU_GATE_UP.
 *
 * dtype: GLU_BF16 or GLU_F16 (GLU_ERR_ENUM for GLU_F32).
 * x, w_gate, w_up must be 16-byte aligned with K, ldx, ldwg, ldwu multiples
 * of 8 elements; h and gu aligned to the element size (GLU_ERR_ARG
 * otherwise).  ldx, ldwg, ldwu >= K and ldh >= N (GLU_ERR_STRIDE).  M, N,
 * K < 2^31, ldx, ldwg, ldwu < 2^24 and at most 2^24 workgroup tiles of
 * 256 x 128 (GLU_ERR_SHAPE).
 * h and gu must not overlap the inputs or each other (GLU_ERR_ALIAS).
 * M == 0 or N == 0 is a no-op; K == 0 gives h = 0.
 */
GLU_API glu_status glu_gemm_fwd(glu_kind kind, glu_dtype dtype, int64_t M, int64_t N, int64_t K,
                        const void *x, int64_t ldx, const void *w_gate, int64_t ldwg,
                        const void *w_up, int64_t ldwu, void *h, int64_t ldh,
                        void *gu, int64_t ldgu, hipStream_t stream);

/*
 * Fused residual add + RMSNorm forward, one row of `hidden` values at a time
 * ("Write a Triton Fused Add+RMSNorm Kernel", Required reasoning process,
 * steps 1-7, and Correctness requirements):
 *   h = x + residual                      (written back: the next residual)
 *   rstd = 1 / sqrt(sum_j h_j^2 / hidden + eps)
 *   y = h * rstd * gamma_j
 * x, residual, h, y: (rows, hidden) with row strides ldx, ldr, ldh, ldy;
 * gamma: (hidden,), contiguous; all of `dtype`.  rstd: (rows,) fp32, or NULL
 * when not needed (training saves it).  eps must be finite and > 0
 * (GLU_ERR_ARG otherwise); it sits inside the square root and the mean
 * divides by `hidden`.  The sum is kept unrounded (fp32 for bf16/fp16, fp64
 * for fp32) for the statistics and y; h is rounded once when stored.
 * h may be exactly x or exactly residual (in-place residual update) and y
 * may be exactly x or residual; h and y must not overlap each other, gamma,
 * rstd, or any input other than exactly.  Rows wider than the kernels'
 * register capacity (65536 bf16/fp16 or 32768 fp32 values on the aligned
 * path) are processed in two passes that re-read x and residual; there h
 * may not overlap x or residual (GLU_ERR_ALIAS).  Forward only.
 */
GLU_API glu_status glu_add_rmsnorm_fwd(glu_dtype dtype, int64_t rows, int64_t hidden,
                               const void *x, int64_t ldx,
                               const void *residual, int64_t ldr,
                               const void *gamma,
                               void *h, int64_t ldh,
                               void *y, int64_t ldy,
                               float *rstd, float eps, hipStream_t stream);

/* Static, NUL-terminated English text for a status code (never NULL). */
GLU_API const char *glu_status_string(glu_status status);

/* Library ABI version: (major << 16) | minor. */
GLU_API int glu_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GLU_H */
