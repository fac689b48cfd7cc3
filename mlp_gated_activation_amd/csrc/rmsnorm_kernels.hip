// rmsnorm_kernels.hip -- gfx950 kernels for the fused residual add + RMSNorm
// forward ("Write a Triton Fused Add+RMSNorm Kernel"):
//   h = x + residual (written back),  rstd = 1/sqrt(mean(h^2) + eps),
//   y = h * rstd * gamma.
//
// One workgroup owns one row (Required reasoning process, step 1).  Every
// thread loads its 16-byte vectors of x, residual and gamma first, forms h in
// fp32 registers (fp64 for fp32 data; step 3), stores h rounded to the storage
// dtype right away (step 4, Kernel design rules), and accumulates sum(h^2).
// The row sum is reduced in a fixed order (wave shuffles, then LDS across the
// waves), rstd is formed once per row (step 5, eps inside the square root,
// denominator H), and y = h * rstd * gamma is stored from the registers
// (steps 6-7): one pass over HBM, 4*H*s bytes per row plus gamma.  Rows wider
// than the register capacity use a two-pass kernel that recomputes h from x
// and residual (step 8, the recompute variant), keeping the arithmetic
// identical.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "glu_internal.h"
#include "rmsnorm_internal.h"

namespace glu {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// vector element -> scalar before any bit_cast (this clang miscompiles
// __builtin_bit_cast applied directly to an ext_vector element)
__device__ inline uint32_t word(u32x4 v, int j)
{
    uint32_t w = v[j];
    return w;
}

struct RBf16 {
    using M = float;
    static constexpr int VE = 8, SIZE = 2;
    __device__ static void unpack(u32x4 v, float *x)
    {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = __builtin_bit_cast(float, word(v, j) << 16);
            x[2 * j + 1] = __builtin_bit_cast(float, word(v, j) & 0xffff0000u);
        }
    }
    __device__ static u32x4 pack(const float *y)
    {
        u32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            v[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{y[2 * j], y[2 * j + 1]}, bf16x2));
        return v;
    }
    __device__ static float load1(const void *p)
    {
        return __builtin_bit_cast(float, uint32_t(*static_cast<const uint16_t *>(p)) << 16);
    }
    __device__ static void store1(void *p, float y) { *static_cast<__bf16 *>(p) = static_cast<__bf16>(y); }
};

struct RF16 {
    using M = float;
    static constexpr int VE = 8, SIZE = 2;
    __device__ static void unpack(u32x4 v, float *x)
    {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f32x2 t = __builtin_convertvector(__builtin_bit_cast(f16x2, word(v, j)), f32x2);
            x[2 * j] = t[0];
            x[2 * j + 1] = t[1];
        }
    }
    __device__ static u32x4 pack(const float *y)
    {
        u32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            v[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{y[2 * j], y[2 * j + 1]}, f16x2));
        return v;
    }
    __device__ static float load1(const void *p) { return float(*static_cast<const _Float16 *>(p)); }
    __device__ static void store1(void *p, float y) { *static_cast<_Float16 *>(p) = static_cast<_Float16>(y); }
};

struct RF32 {
    using M = double;
    static constexpr int VE = 4, SIZE = 4;
    __device__ static void unpack(u32x4 v, double *x)
    {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            x[j] = double(__builtin_bit_cast(float, word(v, j)));
    }
    __device__ static u32x4 pack(const double *y)
    {
        u32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            v[j] = __builtin_bit_cast(uint32_t, float(y[j]));
        return v;
    }
    __device__ static double load1(const void *p) { return double(*static_cast<const float *>(p)); }
    __device__ static void store1(void *p, double y) { *static_cast<float *>(p) = float(y); }
};

#ifndef GLU_RMS_NT_LOAD
#define GLU_RMS_NT_LOAD 1
#endif
#ifndef GLU_RMS_NT_STORE
#define GLU_RMS_NT_STORE 1
#endif
template <typename T> __device__ inline u32x4 ldv(const void *base, int64_t off)
{
    const u32x4 *q = reinterpret_cast<const u32x4 *>(static_cast<const char *>(base) + off * T::SIZE);
#if GLU_RMS_NT_LOAD
    return __builtin_nontemporal_load(q);
#else
    return *q;
#endif
}
template <typename T> __device__ inline u32x4 ldv_cached(const void *base, int64_t off)
{
    // gamma is shared by every row: a normal (cached) load
    return *reinterpret_cast<const u32x4 *>(static_cast<const char *>(base) + off * T::SIZE);
}
template <typename T> __device__ inline void stv(void *base, int64_t off, u32x4 v)
{
    u32x4 *q = reinterpret_cast<u32x4 *>(static_cast<char *>(base) + off * T::SIZE);
#if GLU_RMS_NT_STORE
    __builtin_nontemporal_store(v, q);
#else
    *q = v;
#endif
}
__device__ inline const void *at(const void *b, int64_t off, int size) { return static_cast<const char *>(b) + off * size; }
__device__ inline void *at(void *b, int64_t off, int size) { return static_cast<char *>(b) + off * size; }

__device__ inline float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ inline double shfl_xor(double v, int m) { return __shfl_xor(v, m, 64); }

// Sum over the workgroup in a fixed order: butterfly within each 64-lane wave,
// then the wave totals in wave order.  Every thread returns the total.
template <typename M, int BLOCK> __device__ inline M block_sum(M v, M *lds)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v += shfl_xor(v, m);
    constexpr int NW = BLOCK / 64;
    if constexpr (NW == 1) {
        return v;
    } else {
        const int w = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0)
            lds[w] = v;
        __syncthreads();
        M t = lds[0];
#pragma unroll
        for (int i = 1; i < NW; ++i)
            t += lds[i];
        return t;
    }
}

template <typename M> __device__ inline M rsqrt_row(M ms, float eps) { return M(1) / sqrt(ms + M(eps)); }

// Single pass: VPT vectors per thread stay in registers between the two
// phases.  All register arrays are indexed with compile-time indices only
// (ragged vectors use a guarded, fully unrolled loop), so nothing is demoted
// to scratch memory.  With 8 vectors per thread gamma is loaded in the
// second phase (an L2 hit: every row reads the same gamma), halving the
// registers held across the reduction -- unless GPACK, where its full
// vectors are loaded with the row's first loads and held packed: more
// registers (fewer waves per SIMD), but no wait on gamma between a row's
// reduction and its y stores (rms_gamma_early picks between the two).
template <typename T, int BLOCK, int VPT, bool VEC, bool GPACK = false>
__global__ void __launch_bounds__(BLOCK) add_rmsnorm_kernel(const RmsArgs p)
{
    using M = typename T::M;
    constexpr int VE = VEC ? T::VE : 1;
    constexpr bool G_EARLY = VPT <= 4;
    constexpr bool G_PACK = GPACK && !G_EARLY && VEC;
    __shared__ M lds[BLOCK / 64];
    const int64_t row = blockIdx.x;
    const uint32_t H = p.hidden;
    const void *xr = at(p.x, row * p.ldx, T::SIZE);
    const void *rr = at(p.res, row * p.ldr, T::SIZE);
    void *hr = at(p.h, row * p.ldh, T::SIZE);
    void *yr = at(p.y, row * p.ldy, T::SIZE);

    M h[VPT][VE];
    M g[G_EARLY ? VPT : 1][VE];
    u32x4 gp[G_PACK ? VPT : 1];
    M ss = M(0);
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const uint32_t col = (uint32_t(v) * BLOCK + threadIdx.x) * VE;
        if (VEC && col + VE <= H) {
            M xv[T::VE], rv[T::VE];
            T::unpack(ldv<T>(xr, col), xv);
            T::unpack(ldv<T>(rr, col), rv);
            if constexpr (G_EARLY)
                T::unpack(ldv_cached<T>(p.gamma, col), g[v]);
            if constexpr (G_PACK)
                gp[v] = ldv_cached<T>(p.gamma, col);
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                h[v][e] = xv[e] + rv[e];
                ss += h[v][e] * h[v][e];
            }
            stv<T>(hr, col, T::pack(h[v]));
        } else {
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                if (col + e < H) {
                    M xe = T::load1(at(xr, col + e, T::SIZE));
                    M re = T::load1(at(rr, col + e, T::SIZE));
                    if constexpr (G_EARLY)
                        g[v][e] = T::load1(at(p.gamma, col + e, T::SIZE));
                    h[v][e] = xe + re;
                    ss += h[v][e] * h[v][e];
                    T::store1(at(hr, col + e, T::SIZE), h[v][e]);
                }
            }
        }
    }
    const M rs = rsqrt_row<M>(block_sum<M, BLOCK>(ss, lds) / M(H), p.eps);
    if (p.rstd != nullptr && threadIdx.x == 0)
        p.rstd[row] = float(rs);
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const uint32_t col = (uint32_t(v) * BLOCK + threadIdx.x) * VE;
        if (VEC && col + VE <= H) {
            M gv[T::VE], yv[T::VE];
            if constexpr (G_EARLY) {
#pragma unroll
                for (int e = 0; e < T::VE; ++e)
                    gv[e] = g[v][e];
            } else if constexpr (G_PACK) {
                T::unpack(gp[v], gv);
            } else {
                T::unpack(ldv_cached<T>(p.gamma, col), gv);
            }
#pragma unroll
            for (int e = 0; e < T::VE; ++e)
                yv[e] = h[v][e] * rs * gv[e];
            stv<T>(yr, col, T::pack(yv));
        } else {
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                if (col + e < H) {
                    M ge;
                    if constexpr (G_EARLY)
                        ge = g[v][e];
                    else
                        ge = T::load1(at(p.gamma, col + e, T::SIZE));
                    T::store1(at(yr, col + e, T::SIZE), h[v][e] * rs * ge);
                }
            }
        }
    }
}

// Several rows per workgroup, software-pipelined: the workgroup walks rows
// blockIdx.x, blockIdx.x + gridDim.x, ...; gamma is loaded once and kept in
// registers (packed) for all of them; and the next row's x and residual
// loads are issued as soon as this row's h is formed, before its reduction
// and its y stores, so that each wave always has loads in flight while it
// reduces and stores.  The arithmetic of every row, and the order of its
// sum, are those of the one-row kernel (same BLOCK and VPT), so the results
// are bit-identical.  Vector path only, with H a multiple of the vector
// width (no ragged vector).
template <typename T, int BLOCK, int VPT>
__global__ void __launch_bounds__(BLOCK) add_rmsnorm_rows_kernel(const RmsArgs p, uint32_t rows)
{
    using M = typename T::M;
    constexpr int VE = T::VE;
    constexpr int NW = BLOCK / 64;
    __shared__ M lds[2][NW];
    const uint32_t H = p.hidden;
    uint32_t row = blockIdx.x;
    const uint32_t step = gridDim.x;

    u32x4 gp[VPT], xp[VPT], rp[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const uint32_t col = (uint32_t(v) * BLOCK + threadIdx.x) * VE;
        if (col + VE <= H) {
            gp[v] = ldv_cached<T>(p.gamma, col);
            xp[v] = ldv<T>(at(p.x, int64_t(row) * p.ldx, T::SIZE), col);
            rp[v] = ldv<T>(at(p.res, int64_t(row) * p.ldr, T::SIZE), col);
        }
    }
    for (int parity = 0; row < rows; row += step, parity ^= 1) {
        void *hr = at(p.h, int64_t(row) * p.ldh, T::SIZE);
        void *yr = at(p.y, int64_t(row) * p.ldy, T::SIZE);
        M h[VPT][VE];
        M ss = M(0);
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const uint32_t col = (uint32_t(v) * BLOCK + threadIdx.x) * VE;
            if (col + VE <= H) {
                M xv[VE], rv[VE];
                T::unpack(xp[v], xv);
                T::unpack(rp[v], rv);
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    h[v][e] = xv[e] + rv[e];
                    ss += h[v][e] * h[v][e];
                }
                stv<T>(hr, col, T::pack(h[v]));
            }
        }
        // the next row's loads go out before this row's reduction
        const uint32_t next = row + step;
        if (next < rows) {
            const void *xr = at(p.x, int64_t(next) * p.ldx, T::SIZE);
            const void *rr = at(p.res, int64_t(next) * p.ldr, T::SIZE);
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                const uint32_t col = (uint32_t(v) * BLOCK + threadIdx.x) * VE;
                if (col + VE <= H) {
                    xp[v] = ldv<T>(xr, col);
                    rp[v] = ldv<T>(rr, col);
                }
            }
        }
        // one LDS slot pair per row parity: a wave that runs ahead into the
        // next row cannot overwrite totals another wave still reads, since it
        // would first have to pass that row's barrier
        const M rs = rsqrt_row<M>(block_sum<M, BLOCK>(ss, lds[parity]) / M(H), p.eps);
        if (p.rstd != nullptr && threadIdx.x == 0)
            p.rstd[row] = float(rs);
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const uint32_t col = (uint32_t(v) * BLOCK + threadIdx.x) * VE;
            if (col + VE <= H) {
                M gv[VE], yv[VE];
                T::unpack(gp[v], gv);
#pragma unroll
                for (int e = 0; e < VE; ++e)
                    yv[e] = h[v][e] * rs * gv[e];
                stv<T>(yr, col, T::pack(yv));
            }
        }
    }
}

// Two passes for rows wider than the register capacity: h is recomputed
// from x and residual in the second pass (the host guarantees h aliases
// neither of them).  The first pass reads x and residual through the caches
// (the others stream past them) and the second walks each lane's chunks in
// reverse, so that its re-reads start with what was fetched last; the launch
// keeps one row per CU (kRmsLoopLds), whose 2 x H x s bytes of x and
// residual then stay in the memory-side cache between the passes.
template <typename T, int BLOCK, bool VEC>
__global__ void __launch_bounds__(BLOCK) add_rmsnorm_loop_kernel(const RmsArgs p)
{
    using M = typename T::M;
    constexpr int VE = VEC ? T::VE : 1;
    __shared__ M lds[BLOCK / 64];
    const int64_t row = blockIdx.x;
    const uint32_t H = p.hidden;
    const void *xr = at(p.x, row * p.ldx, T::SIZE);
    const void *rr = at(p.res, row * p.ldr, T::SIZE);
    void *hr = at(p.h, row * p.ldh, T::SIZE);
    void *yr = at(p.y, row * p.ldy, T::SIZE);
    M ss = M(0);
    for (uint32_t col = threadIdx.x * VE; col < H; col += uint32_t(BLOCK) * VE) {
        M hv[T::VE];
        if (VEC && col + VE <= H) {
            M xv[T::VE], rv[T::VE];
            T::unpack(ldv_cached<T>(xr, col), xv);
            T::unpack(ldv_cached<T>(rr, col), rv);
#pragma unroll
            for (int e = 0; e < T::VE; ++e) {
                hv[e] = xv[e] + rv[e];
                ss += hv[e] * hv[e];
            }
            stv<T>(hr, col, T::pack(hv));
        } else {
            const uint32_t n = H - col < uint32_t(VE) ? H - col : uint32_t(VE);
            for (uint32_t e = 0; e < n; ++e) {
                M he = T::load1(at(xr, col + e, T::SIZE)) + T::load1(at(rr, col + e, T::SIZE));
                ss += he * he;
                T::store1(at(hr, col + e, T::SIZE), he);
            }
        }
    }
    const M rs = rsqrt_row<M>(block_sum<M, BLOCK>(ss, lds) / M(H), p.eps);
    if (p.rstd != nullptr && threadIdx.x == 0)
        p.rstd[row] = float(rs);
    const uint32_t c0 = threadIdx.x * VE, stride = uint32_t(BLOCK) * VE;
    const int64_t nlast = c0 < H ? int64_t((H - 1 - c0) / stride) : -1;
    for (int64_t i = nlast; i >= 0; --i) {
        const uint32_t col = c0 + uint32_t(i) * stride;
        if (VEC && col + VE <= H) {
            M xv[T::VE], rv[T::VE], gv[T::VE], yv[T::VE];
            T::unpack(ldv<T>(xr, col), xv);
            T::unpack(ldv<T>(rr, col), rv);
            T::unpack(ldv_cached<T>(p.gamma, col), gv);
#pragma unroll
            for (int e = 0; e < T::VE; ++e)
                yv[e] = (xv[e] + rv[e]) * rs * gv[e];
            stv<T>(yr, col, T::pack(yv));
        } else {
            const uint32_t n = H - col < uint32_t(VE) ? H - col : uint32_t(VE);
            for (uint32_t e = 0; e < n; ++e) {
                M he = T::load1(at(xr, col + e, T::SIZE)) + T::load1(at(rr, col + e, T::SIZE));
                T::store1(at(yr, col + e, T::SIZE), he * rs * T::load1(at(p.gamma, col + e, T::SIZE)));
            }
        }
    }
}

typedef void (*RmsFn)(const RmsArgs);
typedef void (*RmsRowsFn)(const RmsArgs, uint32_t);

// Pipelined instances for the single-pass shapes of the default table with
// at most 4 vectors per thread and 512 threads (the others keep the one-row
// kernel: holding the next row on top of this one, their fp32-data
// instances spill, at 8 vectors per thread or under the 128-register limit
// of 1024-thread workgroups).
template <typename T> RmsRowsFn pick_rms_rows(RmsShape s)
{
    switch (s.block * 16 + s.vpt) {
    case 64 * 16 + 1: return &add_rmsnorm_rows_kernel<T, 64, 1>;
    case 64 * 16 + 2: return &add_rmsnorm_rows_kernel<T, 64, 2>;
    case 64 * 16 + 4: return &add_rmsnorm_rows_kernel<T, 64, 4>;
    case 256 * 16 + 4: return &add_rmsnorm_rows_kernel<T, 256, 4>;
    case 512 * 16 + 4: return &add_rmsnorm_rows_kernel<T, 512, 4>;
    }
    return nullptr;
}

template <typename T, bool VEC> RmsFn pick_rms(RmsShape s)
{
    if (s.vpt == 0)
        return &add_rmsnorm_loop_kernel<T, kRmsLoopBlock, VEC>;
    switch (s.block * 16 + s.vpt) {
    case 64 * 16 + 1: return &add_rmsnorm_kernel<T, 64, 1, VEC>;
    case 64 * 16 + 2: return &add_rmsnorm_kernel<T, 64, 2, VEC>;
    case 64 * 16 + 4: return &add_rmsnorm_kernel<T, 64, 4, VEC>;
    case 64 * 16 + 8: return &add_rmsnorm_kernel<T, 64, 8, VEC>;
    case 128 * 16 + 4: return &add_rmsnorm_kernel<T, 128, 4, VEC>;
    case 128 * 16 + 8: return &add_rmsnorm_kernel<T, 128, 8, VEC>;
    case 512 * 16 + 4: return &add_rmsnorm_kernel<T, 512, 4, VEC>;
    case 1024 * 16 + 4: return &add_rmsnorm_kernel<T, 1024, 4, VEC>;
    case 128 * 16 + 1: return &add_rmsnorm_kernel<T, 128, 1, VEC>;
    case 256 * 16 + 1: return &add_rmsnorm_kernel<T, 256, 1, VEC>;
    case 256 * 16 + 2: return &add_rmsnorm_kernel<T, 256, 2, VEC>;
    case 256 * 16 + 4: return &add_rmsnorm_kernel<T, 256, 4, VEC>;
    case 256 * 16 + 8: return &add_rmsnorm_kernel<T, 256, 8, VEC>;
    case 512 * 16 + 8: return &add_rmsnorm_kernel<T, 512, 8, VEC>;
    case 1024 * 16 + 8: return &add_rmsnorm_kernel<T, 1024, 8, VEC>;
    }
    return nullptr;
}

template <typename T> RmsFn pick_rms_vec(bool vec, RmsShape s)
{
    return vec ? pick_rms<T, true>(s) : pick_rms<T, false>(s);
}

// Rows of the 64-thread, 8-vector shape one CU holds at once, four SIMDs
// times the waves per SIMD its registers allow: <= 96 VGPRs (five waves)
// with gamma loaded late, 97 .. 128 (four) with it early and packed.  The
// kernel ISA test checks the compiled register counts against both.
constexpr int64_t kRmsRowsPerCuLate = 20, kRmsRowsPerCuEarly = 16;

// The early-gamma instance when the rows take more than one round of the
// late one and no more rounds of the early one.  bf16, 4096 wide, early
// against late, same process, bit-identical: 6144 rows 38.1 / 41.3 us, 8192
// 48.6 / 51.4, 12288 71.8 / 73.6, 16384 93.8 / 96.9 (and 8192 x 3072 37.2 /
// 39.4); within one round even (4096 rows 23.99 / 23.93), so the late one
// stays there; and 5120 rows 33.5 / 29.6, where the early one needs a
// second round.
bool rms_gamma_early(uint32_t rows, hipStream_t stream)
{
    int dev = 0, cus = 0;
    if ((stream != nullptr ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev)) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return false;
    const int64_t se = kRmsRowsPerCuEarly * cus, sl = kRmsRowsPerCuLate * cus;
    return int64_t(rows) > sl && (int64_t(rows) + se - 1) / se == (int64_t(rows) + sl - 1) / sl;
}

}  // namespace

hipError_t launch_add_rmsnorm(int dtype, bool vec, RmsShape shape, uint32_t rows, const RmsArgs &args,
                              hipStream_t stream)
{
    RmsArgs copy = args;
    const int ve = dtype == F32 ? 4 : 8;
    if (shape.rpb > 1 && vec && shape.vpt > 0 && args.hidden % uint32_t(ve) == 0) {
        RmsRowsFn rf = dtype == F32 ? pick_rms_rows<RF32>(shape)
                     : dtype == F16 ? pick_rms_rows<RF16>(shape)
                                    : pick_rms_rows<RBf16>(shape);
        if (rf != nullptr) {
            uint32_t nrows = rows;
            void *rargs[] = {&copy, &nrows};
            const uint32_t grid = (rows + uint32_t(shape.rpb) - 1) / uint32_t(shape.rpb);
            return hipLaunchKernel(reinterpret_cast<const void *>(rf), dim3(grid), dim3(shape.block), rargs, 0,
                                   stream);
        }
    }
    RmsFn fn = dtype == F32 ? pick_rms_vec<RF32>(vec, shape)
             : dtype == F16 ? pick_rms_vec<RF16>(vec, shape)
                            : pick_rms_vec<RBf16>(vec, shape);
    if (vec && dtype != F32 && shape.block == 64 && shape.vpt == 8 && rms_gamma_early(rows, stream))
        fn = dtype == F16 ? &add_rmsnorm_kernel<RF16, 64, 8, true, true> : &add_rmsnorm_kernel<RBf16, 64, 8, true, true>;
    if (fn == nullptr)
        return hipErrorInvalidConfiguration;
    void *kargs[] = {&copy};
    // The two-pass kernel reserves LDS it does not use, which keeps one row
    // (workgroup) per CU: bf16 4096 x 131072 3789 -> 4949 GB/s together with
    // the cached first pass and the reversed second pass, 2048 x 70000 3418
    // -> 4735.
    constexpr unsigned kRmsLoopLds = 96 * 1024;
    return hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3(rows), dim3(shape.block), kargs,
                           shape.vpt == 0 ? kRmsLoopLds : 0, stream);
}

}  // namespace glu
