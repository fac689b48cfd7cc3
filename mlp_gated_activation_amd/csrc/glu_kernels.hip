// glu_kernels.hip -- gfx950 kernels for y = act(a) * b and its backward.
//
// Sources (page title -- section):
//   [SWIGLU] "Write a Triton SiLU-Mul (SwiGLU) Kernel"
//   [LIGER]  "Kernel Profile: SwiGLU (Tier 1 -- Element-wise)"
//   [FUSED]  "Fused Kernels"
//
// The op is a pure elementwise stream: 2 loads + 1 store per element forward,
// 3 loads + 2 stores backward, a handful of fp32 operations in between
// ([SWIGLU] "Performance requirements": arithmetic intensity well under one
// flop per byte).  So the design is all about HBM:
//  - each lane moves whole 16-byte vectors of every stream (global_load_dwordx4
//    / global_store_dwordx4), and a wave covers 1 KiB contiguous per stream;
//  - all of a thread's loads are issued before any math, so GLU_UNROLL
//    vectors per stream are in flight per lane;
//  - loads and stores carry the non-temporal hint: nothing is reused;
//  - rows are addressed through row strides with one multiply-high division
//    per 16-byte unit, never a per-element divide ([SWIGLU] "Performance
//    requirements", interleaved layout cost);
//  - there is no LDS traffic, no cross-lane traffic and no MFMA (the light
//    16-bit kinds reserve LDS only to cap the workgroups per CU; see launch).
// Math: bf16/fp16 are widened to fp32, fp32 to fp64; the result is rounded
// once at the store ([SWIGLU] "Kernel design rules").
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "glu_act.h"
#include "glu_internal.h"

namespace glu {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));


// ---------------------------------------------------------------------------
// Storage types: unpack a 16-byte vector to the math type, pack it back with
// one round-to-nearest-even per element.
//
// word() copies a vector element into a scalar before any __builtin_bit_cast:
// this clang miscompiles __builtin_bit_cast applied directly to an
// ext_vector element (it reads element 0 for every index).
// ---------------------------------------------------------------------------
__device__ inline uint32_t word(u32x4 v, int j)
{
    uint32_t w = v[j];
    return w;
}

struct SBf16 {
    using M = float;
    static constexpr int VE = 8;
    static constexpr int SIZE = 2;
    static constexpr bool PATCH = false;
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

struct SF16 {
    using M = float;
    static constexpr int VE = 8;
    static constexpr int SIZE = 2;
    static constexpr bool PATCH = true;   // fp16 inputs reach within 2e-5 of act''s root
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

struct SF32 {
    using M = double;
    static constexpr int VE = 4;
    static constexpr int SIZE = 4;
    static constexpr bool PATCH = false;
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


// ---------------------------------------------------------------------------
// The kernel.  Unit u of the launch covers row r = u / units_per_row and
// columns [j*VE, min(j*VE + VE, cols)), j = u - r*units_per_row.  A unit
// that reaches past the row end (cols not a multiple of VE) is handled
// element by element; no access ever leaves [0, cols) of a row
// ([SWIGLU] "Kernel design rules": always mask the tail).
// ---------------------------------------------------------------------------
template <typename T>
__device__ inline u32x4 ldv(const void *base, int64_t off_elems)
{
    const u32x4 *p = reinterpret_cast<const u32x4 *>(static_cast<const char *>(base) + off_elems * T::SIZE);
#if GLU_NT_LOAD
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

template <typename T>
__device__ inline void stv(void *base, int64_t off_elems, u32x4 v)
{
    u32x4 *p = reinterpret_cast<u32x4 *>(static_cast<char *>(base) + off_elems * T::SIZE);
#if GLU_NT_STORE
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

__device__ inline const void *at(const void *base, int64_t off, int size)
{
    return static_cast<const char *>(base) + off * size;
}
__device__ inline void *at(void *base, int64_t off, int size) { return static_cast<char *>(base) + off * size; }

template <typename T, int KIND, bool BWD, bool VEC, bool FLAT, int BLOCK>
__global__ void __launch_bounds__(BLOCK) glu_kernel(const Args p)
{
    using M = typename T::M;
    constexpr int VE = VEC ? T::VE : 1;
    constexpr int U = GLU_UNROLL;

#if GLU_XCD_REMAP
    // Blocks are dispatched round-robin over the 8 XCDs; give XCD x the
    // x-th contiguous eighth of the blocks (when the grid divides evenly).
    uint32_t bid = blockIdx.x;
    if ((gridDim.x & 7u) == 0)
        bid = (bid & 7u) * (gridDim.x >> 3) + (bid >> 3);
    const uint32_t first = bid * uint32_t(BLOCK * U) + threadIdx.x;
#else
    const uint32_t first = blockIdx.x * uint32_t(BLOCK * U) + threadIdx.x;
#endif

    uint32_t row[U], col[U];
    bool live[U], full[U];
    u32x4 va[U], vb[U], vd[U];

    // Phase 1: locate every unit and issue all full-vector loads.
#pragma unroll
    for (int k = 0; k < U; ++k) {
        uint32_t u = first + uint32_t(k * BLOCK);
        live[k] = u < p.units;
        // FLAT: the launch is a single row (dense operands merged), no division
        uint32_t r = FLAT ? 0u : (__umulhi(u, p.row_div.magic) + u) >> p.row_div.shift;
        row[k] = r;
        col[k] = (u - r * p.units_per_row) * uint32_t(VE);
        full[k] = live[k] && (col[k] + uint32_t(VE) <= p.cols);
        if constexpr (VEC) {
            if (full[k]) {
                va[k] = ldv<T>(p.in0, int64_t(r) * p.ld_in0 + col[k]);
                vb[k] = ldv<T>(p.in1, int64_t(r) * p.ld_in1 + col[k]);
                if constexpr (BWD)
                    vd[k] = ldv<T>(p.in2, int64_t(r) * p.ld_in2 + col[k]);
            }
        }
    }

    // Phase 2: compute and store.
#pragma unroll
    for (int k = 0; k < U; ++k) {
        if (!live[k])
            continue;
        const int64_t r = row[k];
        if (VEC && full[k]) {
            M a[T::VE], b[T::VE], o0[T::VE];
            T::unpack(va[k], a);
            T::unpack(vb[k], b);
            if constexpr (!BWD) {
#pragma unroll
                for (int e = 0; e < T::VE; ++e)
                    o0[e] = act<KIND, M>(a[e]) * b[e];
                stv<T>(p.out0, r * p.ld_out0 + col[k], T::pack(o0));
            } else {
                M dy[T::VE], o1[T::VE];
                T::unpack(vd[k], dy);
#pragma unroll
                for (int e = 0; e < T::VE; ++e) {
                    M f, g;
                    act_grad<KIND, T::PATCH, M>(a[e], f, g);
                    o0[e] = (dy[e] * g) * b[e];
                    o1[e] = dy[e] * f;
                }
                stv<T>(p.out0, r * p.ld_out0 + col[k], T::pack(o0));
                stv<T>(p.out1, r * p.ld_out1 + col[k], T::pack(o1));
            }
        } else {
            // element path: unaligned data, or the ragged end of a row
            const uint32_t n = p.cols - col[k] < uint32_t(VE) ? p.cols - col[k] : uint32_t(VE);
            for (uint32_t e = 0; e < n; ++e) {
                const int64_t c = int64_t(col[k]) + e;
                M a = T::load1(at(p.in0, r * p.ld_in0 + c, T::SIZE));
                M b = T::load1(at(p.in1, r * p.ld_in1 + c, T::SIZE));
                if constexpr (!BWD) {
                    T::store1(at(p.out0, r * p.ld_out0 + c, T::SIZE), act<KIND, M>(a) * b);
                } else {
                    M dy = T::load1(at(p.in2, r * p.ld_in2 + c, T::SIZE));
                    M f, g;
                    act_grad<KIND, T::PATCH, M>(a, f, g);
                    T::store1(at(p.out0, r * p.ld_out0 + c, T::SIZE), (dy * g) * b);
                    T::store1(at(p.out1, r * p.ld_out1 + c, T::SIZE), dy * f);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Tiled kernel for strided operands of mixed layouts.  One workgroup of 256
// threads (4 waves) owns a 64 x 64 tile and computes it in row orientation:
// thread chunk q = tid + 256*j (j < CPT) is line q / LINE, segment q % LINE,
// i.e. the VE elements (line, seg*VE + e).
//  - kDirect operands (column stride 1) move those chunks straight between
//    HBM and registers as 16-byte vectors;
//  - kTransposed operands (row stride 1) move 16-byte chunks down a column,
//    (seg*VE + e, line), and are turned around through LDS: float slots with
//    a row pitch of 65 words, which is conflict-free both ways;
//  - kGather operands are read / written element by element.
// Every load of the tile is issued before any LDS traffic or math.  Values
// are exact in float (the fp32 data's compute widening to double happens in
// registers); results are rounded once to the storage type.
// ---------------------------------------------------------------------------
template <typename T> __device__ inline void unpack_f(u32x4 v, float *x)
{
    if constexpr (T::SIZE == 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            x[j] = __builtin_bit_cast(float, word(v, j));
    } else {
        T::unpack(v, x);
    }
}
template <typename T> __device__ inline u32x4 pack_f(const float *y)
{
    if constexpr (T::SIZE == 4) {
        u32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            v[j] = __builtin_bit_cast(uint32_t, y[j]);
        return v;
    } else {
        return T::pack(y);
    }
}

template <typename T, int KIND, bool BWD>
__global__ void __launch_bounds__(256) glu_tile_kernel(const TileArgs p)
{
    using M = typename T::M;
    constexpr int NIN = BWD ? 3 : 2, NOUT = BWD ? 2 : 1;
    constexpr int VE = T::VE;                             // elements per 16-byte chunk
    constexpr int LINE = kTile / VE;                      // chunks per tile line
    constexpr int CPT = kTile * kTile / (256 * VE);       // chunks per thread
    // nslots slots of kTile x (kTile + 1) floats, sized at launch
    extern __shared__ float lds_raw[];
    float(*lds)[kTile][kTile + 1] = reinterpret_cast<float(*)[kTile][kTile + 1]>(lds_raw);

    const TileCoord tc = tile_coord(p.tile0 + blockIdx.x, p.tiles_r, p.tiles_c);
    const int64_t r0 = int64_t(tc.r) * kTile, c0 = int64_t(tc.c) * kTile;
    const int tid = threadIdx.x;

    // Phase 1: every full 16-byte chunk of every input, all loads in flight.
    u32x4 raw[NIN][CPT];
    bool vec[NIN][CPT];
#pragma unroll
    for (int k = 0; k < NIN; ++k) {
        const int mode = p.in_mode[k];
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int q = tid + 256 * j, line = q / LINE, seg = q % LINE;
            const bool tr = mode == kTransposed;
            const int64_t r = tr ? r0 + seg * VE : r0 + line, c = tr ? c0 + line : c0 + seg * VE;
            vec[k][j] = mode != kGather && (tr ? (c < p.cols && r + VE <= p.rows) : (r < p.rows && c + VE <= p.cols));
            if (vec[k][j])
                raw[k][j] = ldv<T>(p.in[k], r * p.irs[k] + c * p.ics[k]);
        }
    }
    // Unpack, or fetch element by element (gathered operands, ragged edges;
    // outside the problem: 0).
    float x[NIN][CPT][VE];
#pragma unroll
    for (int k = 0; k < NIN; ++k) {
        const bool tr = p.in_mode[k] == kTransposed;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            if (vec[k][j]) {
                unpack_f<T>(raw[k][j], x[k][j]);
            } else {
                const int q = tid + 256 * j, line = q / LINE, seg = q % LINE;
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    const int64_t r = tr ? r0 + seg * VE + e : r0 + line;
                    const int64_t c = tr ? c0 + line : c0 + seg * VE + e;
                    x[k][j][e] = (r < p.rows && c < p.cols)
                                     ? float(T::load1(at(p.in[k], r * p.irs[k] + c * p.ics[k], T::SIZE)))
                                     : 0.0f;
                }
            }
        }
    }

    // Phase 2: turn the transposed inputs around through LDS.
#pragma unroll
    for (int k = 0; k < NIN; ++k)
        if (p.in_mode[k] == kTransposed) {
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                const int q = tid + 256 * j, line = q / LINE, seg = q % LINE;
#pragma unroll
                for (int e = 0; e < VE; ++e)
                    lds[p.in_slot[k]][seg * VE + e][line] = x[k][j][e];
            }
        }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NIN; ++k)
        if (p.in_mode[k] == kTransposed) {
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                const int q = tid + 256 * j, line = q / LINE, seg = q % LINE;
#pragma unroll
                for (int e = 0; e < VE; ++e)
                    x[k][j][e] = lds[p.in_slot[k]][line][seg * VE + e];
            }
        }

    // Phase 3: the math, in row orientation; one rounding per result.
    float y[NOUT][CPT][VE];
#pragma unroll
    for (int j = 0; j < CPT; ++j)
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            const M a = M(x[0][j][e]), b = M(x[1][j][e]);
            if constexpr (!BWD) {
                y[0][j][e] = float(act<KIND, M>(a) * b);
            } else {
                const M dy = M(x[2][j][e]);
                M f, g;
                act_grad<KIND, T::PATCH, M>(a, f, g);
                y[0][j][e] = float((dy * g) * b);
                y[1][j][e] = float(dy * f);
            }
        }

    // Phase 4: transposed outputs go back through LDS, then every output is
    // stored along its own contiguous direction.
    __syncthreads();   // phase-2 reads are done before the slots are reused
#pragma unroll
    for (int k = 0; k < NOUT; ++k)
        if (p.out_mode[k] == kTransposed) {
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                const int q = tid + 256 * j, line = q / LINE, seg = q % LINE;
#pragma unroll
                for (int e = 0; e < VE; ++e)
                    lds[p.out_slot[k]][line][seg * VE + e] = y[k][j][e];
            }
        }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NOUT; ++k) {
        const int mode = p.out_mode[k];
        const bool tr = mode == kTransposed;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int q = tid + 256 * j, line = q / LINE, seg = q % LINE;
            float v[VE];
            if (tr) {
#pragma unroll
                for (int e = 0; e < VE; ++e)
                    v[e] = lds[p.out_slot[k]][seg * VE + e][line];
            } else {
#pragma unroll
                for (int e = 0; e < VE; ++e)
                    v[e] = y[k][j][e];
            }
            const int64_t r = tr ? r0 + seg * VE : r0 + line, c = tr ? c0 + line : c0 + seg * VE;
            const bool full = mode != kGather && (tr ? (c < p.cols && r + VE <= p.rows) : (r < p.rows && c + VE <= p.cols));
            if (full) {
                stv<T>(p.out[k], r * p.ors[k] + c * p.ocs[k], pack_f<T>(v));
            } else {
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    const int64_t rr = tr ? r + e : r, cc = tr ? c : c + e;
                    if (rr < p.rows && cc < p.cols)
                        T::store1(at(p.out[k], rr * p.ors[k] + cc * p.ocs[k], T::SIZE), M(v[e]));
                }
            }
        }
    }
}

typedef void (*TileFn)(const TileArgs);

template <typename T, bool BWD> TileFn pick_tile(int kind)
{
    switch (kind) {
    case SILU: return &glu_tile_kernel<T, SILU, BWD>;
    case GELU_ERF: return &glu_tile_kernel<T, GELU_ERF, BWD>;
    case GELU_TANH: return &glu_tile_kernel<T, GELU_TANH, BWD>;
    default: return &glu_tile_kernel<T, RELU, BWD>;
    }
}

// ---------------------------------------------------------------------------
// Dispatch table: [dtype][kind][backward][vec].
// ---------------------------------------------------------------------------
typedef void (*KernelFn)(const Args);

template <typename T, int KIND, bool BWD, int BLOCK>
constexpr KernelFn pick(bool vec, bool flat)
{
    return vec ? (flat ? &glu_kernel<T, KIND, BWD, true, true, BLOCK> : &glu_kernel<T, KIND, BWD, true, false, BLOCK>)
               : (flat ? &glu_kernel<T, KIND, BWD, false, true, BLOCK> : &glu_kernel<T, KIND, BWD, false, false, BLOCK>);
}

// The forward has one block size; the backward a large-launch and a
// small-launch one.
template <typename T, int KIND>
KernelFn pick_dir(bool bwd, bool small, bool vec, bool flat)
{
    if (!bwd)
        return pick<T, KIND, false, GLU_BLOCK_FWD>(vec, flat);
    return small ? pick<T, KIND, true, GLU_BLOCK_BWD_SMALL>(vec, flat) : pick<T, KIND, true, GLU_BLOCK_BWD>(vec, flat);
}

template <typename T>
KernelFn pick_kind(int kind, bool bwd, bool small, bool vec, bool flat)
{
    switch (kind) {
    case SILU: return pick_dir<T, SILU>(bwd, small, vec, flat);
    case GELU_ERF: return pick_dir<T, GELU_ERF>(bwd, small, vec, flat);
    case GELU_TANH: return pick_dir<T, GELU_TANH>(bwd, small, vec, flat);
    default: return pick_dir<T, RELU>(bwd, small, vec, flat);
    }
}

}  // namespace

hipError_t launch_tiles(int dtype, int kind, bool backward, const TileArgs &args, uint32_t ntiles,
                        hipStream_t stream)
{
    TileFn fn = dtype == F32 ? (backward ? pick_tile<SF32, true>(kind) : pick_tile<SF32, false>(kind))
              : dtype == F16 ? (backward ? pick_tile<SF16, true>(kind) : pick_tile<SF16, false>(kind))
                             : (backward ? pick_tile<SBf16, true>(kind) : pick_tile<SBf16, false>(kind));
    TileArgs copy = args;
    void *kargs[] = {&copy};
    // The slots the launch needs, but at least kTileMinLds: that caps the
    // tiled kernels at five workgroups per CU.  The forward kernels' register
    // count would allow eight, and the extra tiles in flight only slow the
    // transposed stores (forward into a transposed y at 4096 x 14336 bf16:
    // 4754 GB/s uncapped, 5397 at five per CU, 3695 at two); the backward
    // kernels' registers already cap them at four.
    constexpr size_t kTileMinLds = 32 * 1024;
    size_t lds = size_t(args.nslots) * kTile * (kTile + 1) * sizeof(float);
    lds = lds < kTileMinLds ? kTileMinLds : lds;
    return hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3(ntiles), dim3(256), kargs, lds, stream);
}

hipError_t launch(int dtype, int kind, bool backward, bool vec, const Args &args, hipStream_t stream)
{
    // a launch whose units all lie in one row needs no row division
    const bool flat = args.units == args.units_per_row;
    const bool small = args.units < kCapMinUnits;
    KernelFn fn = dtype == F32 ? pick_kind<SF32>(kind, backward, small, vec, flat)
                : dtype == F16 ? pick_kind<SF16>(kind, backward, small, vec, flat)
                               : pick_kind<SBf16>(kind, backward, small, vec, flat);
    const uint32_t bs = !backward ? GLU_BLOCK_FWD : small ? GLU_BLOCK_BWD_SMALL : GLU_BLOCK_BWD;
    const uint32_t per_block = bs * GLU_UNROLL;
    dim3 grid((args.units + per_block - 1) / per_block);
    dim3 block(bs);
    Args copy = args;
    void *kargs[] = {&copy};
    // The kernels use no LDS; on 16-bit data, reserving some caps the
    // workgroups resident on a CU (160 KiB of LDS each): 25 forward (64
    // threads), 10 backward (128 threads).  Fewer streams in flight per CU
    // moved more bytes on MI355X: bf16 SwiGLU 4096 x 14336 fwd 6521 -> 6643
    // GB/s, bwd 6380 -> 6470; fp16 [gate | up] 8191 x 18944 ReGLU fwd 6702 ->
    // 6783, bwd 6466 -> 6602; and, with inputs restored between timed
    // batches, the GELU kinds 1-2.5 % in both directions (bf16 4096 x 14336
    // GELU-erf fwd 6399 -> 6515, bwd 6341 -> 6408; fp16 [gate | up] 8191 x
    // 18944 GELU-erf fwd 6639 -> 6808, bwd 6434 -> 6552; GELU-tanh alike).
    // At 24 forward workgroups per CU the forward falls back.  fp32 data
    // (fp64 arithmetic) lost up to 8 % capped and keeps every workgroup it
    // can.  Small launches, too: below 2^22 units (4096 x 8192 bf16) the cap
    // leaves a second, partial round of workgroups, and uncapped they ran
    // 2-3.5 % faster at 4096 x 512 .. 3072 (even at 4096 x 4096 .. 6144),
    // while the cap gained 1 % from 4096 x 8192 up.
    const bool cap = dtype != F32 && args.units >= kCapMinUnits;
    const unsigned lds = !cap ? 0u : backward ? kCapLdsBwd : kCapLdsFwd;
    return hipLaunchKernel(reinterpret_cast<const void *>(fn), grid, block, kargs, lds, stream);
}

}  // namespace glu
