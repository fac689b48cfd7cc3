// stream_ref.hip -- data-movement reference kernels (include/glu_ref.h).
//
// Measurement infrastructure, not part of the method: the mix kernels move
// the bytes of one streaming gated-activation launch with the same
// per-thread access (one 16-byte non-temporal vector per stream), the same
// workgroup size and the same LDS reservation that caps resident workgroups
// per CU, and replace the arithmetic by an XOR; the RMSNorm mix moves the
// fused add + RMSNorm forward's bytes as a flat stream; the tiled mixes move
// the strided kernels' bytes in their 64 x 64 tile pattern.  Built into its own
// library so the method's library exports only the method's entry points.
#include "glu_ref.h"
#include "glu_internal.h"

#include <hip/hip_runtime.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One launch covers fewer than 2^31 vectors, so 32-bit indices never wrap.
constexpr uint64_t kMaxVecs = uint64_t(1) << 30;

template <int BLOCK>
__global__ void __launch_bounds__(BLOCK) fwd_mix_kernel(const u32x4 *a, const u32x4 *b, u32x4 *y, uint32_t n)
{
    const uint32_t i = blockIdx.x * uint32_t(BLOCK) + threadIdx.x;
    if (i >= n)
        return;
    const u32x4 va = __builtin_nontemporal_load(a + i);
    const u32x4 vb = __builtin_nontemporal_load(b + i);
    __builtin_nontemporal_store(va ^ vb, y + i);
}

template <int BLOCK>
__global__ void __launch_bounds__(BLOCK) bwd_mix_kernel(const u32x4 *a, const u32x4 *b, const u32x4 *d, u32x4 *da,
                                                        u32x4 *db, uint32_t n)
{
    const uint32_t i = blockIdx.x * uint32_t(BLOCK) + threadIdx.x;
    if (i >= n)
        return;
    const u32x4 va = __builtin_nontemporal_load(a + i);
    const u32x4 vb = __builtin_nontemporal_load(b + i);
    const u32x4 vd = __builtin_nontemporal_load(d + i);
    __builtin_nontemporal_store(va ^ vd, da + i);
    __builtin_nontemporal_store(vb ^ vd, db + i);
}

__global__ void __launch_bounds__(64) rms_mix_kernel(const u32x4 *x, const u32x4 *r, u32x4 *h, u32x4 *y, uint32_t n)
{
    const uint32_t i = blockIdx.x * 64u + threadIdx.x;
    if (i >= n)
        return;
    const u32x4 vx = __builtin_nontemporal_load(x + i);
    const u32x4 vr = __builtin_nontemporal_load(r + i);
    __builtin_nontemporal_store(vx ^ vr, h + i);
    __builtin_nontemporal_store(vx + vr, y + i);
}

// Tiled mixes: chunk q = tid + 256 j of a 64 x 64 bf16 tile is row-major
// line q / 8, segment q % 8 (8 elements); the transposed operand's chunk q is
// column q / 8, rows 8 (q % 8) .. + 7, turned around through LDS as floats.
constexpr int kT = 64;
__device__ inline float lo16(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ inline float hi16(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
__device__ inline uint32_t join16(float lo, float hi)
{
    return (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xffff0000u);
}

__global__ void __launch_bounds__(256) tile_bwd_mix_kernel(const uint16_t *a, const uint16_t *b, const uint16_t *dyT,
                                                           uint16_t *da, uint16_t *db, int64_t rows, int64_t cols,
                                                           uint32_t tiles_r, uint32_t tiles_c)
{
    __shared__ float lds[kT][kT + 1];
    const glu::TileCoord tc = glu::tile_coord(blockIdx.x, tiles_r, tiles_c);
    const int64_t r0 = int64_t(tc.r) * kT, c0 = int64_t(tc.c) * kT;
    u32x4 va[2], vb[2], vd[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int q = threadIdx.x + 256 * j, line = q / 8, seg = q % 8;
        va[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a + (r0 + line) * cols + c0 + seg * 8));
        vb[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(b + (r0 + line) * cols + c0 + seg * 8));
        vd[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(dyT + (c0 + line) * rows + r0 + seg * 8));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int q = threadIdx.x + 256 * j, line = q / 8, seg = q % 8;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t w = vd[j][e];
            lds[seg * 8 + 2 * e][line] = lo16(w);
            lds[seg * 8 + 2 * e + 1][line] = hi16(w);
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int q = threadIdx.x + 256 * j, line = q / 8, seg = q % 8;
        u32x4 d;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            d[e] = join16(lds[line][seg * 8 + 2 * e], lds[line][seg * 8 + 2 * e + 1]);
        __builtin_nontemporal_store(va[j] ^ d, reinterpret_cast<u32x4 *>(da + (r0 + line) * cols + c0 + seg * 8));
        __builtin_nontemporal_store(vb[j] ^ d, reinterpret_cast<u32x4 *>(db + (r0 + line) * cols + c0 + seg * 8));
    }
}

__global__ void __launch_bounds__(256) tile_fwd_mix_kernel(const uint16_t *a, const uint16_t *b, uint16_t *yT,
                                                           int64_t rows, int64_t cols, uint32_t tiles_r,
                                                           uint32_t tiles_c)
{
    __shared__ float lds[kT][kT + 1];
    const glu::TileCoord tc = glu::tile_coord(blockIdx.x, tiles_r, tiles_c);
    const int64_t r0 = int64_t(tc.r) * kT, c0 = int64_t(tc.c) * kT;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int q = threadIdx.x + 256 * j, line = q / 8, seg = q % 8;
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a + (r0 + line) * cols + c0 + seg * 8)) ^
                        __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(b + (r0 + line) * cols + c0 + seg * 8));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t w = v[e];
            lds[line][seg * 8 + 2 * e] = lo16(w);
            lds[line][seg * 8 + 2 * e + 1] = hi16(w);
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int q = threadIdx.x + 256 * j, line = q / 8, seg = q % 8;
        u32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            y[e] = join16(lds[seg * 8 + 2 * e][line], lds[seg * 8 + 2 * e + 1][line]);
        __builtin_nontemporal_store(y, reinterpret_cast<u32x4 *>(yT + (c0 + line) * rows + r0 + seg * 8));
    }
}

// 48 KiB per workgroup in all (the static tile plus this), three per CU.
constexpr unsigned kTileMixDynLds = 48 * 1024 - kT * (kT + 1) * 4;

bool tile_shape_ok(int64_t rows, int64_t cols)
{
    return rows > 0 && cols > 0 && rows % kT == 0 && cols % kT == 0 &&
           (rows / kT) * (cols / kT) <= int64_t(glu::kMaxTilesPerLaunch);
}

__global__ void __launch_bounds__(256) copy_kernel(const u32x4 *s, u32x4 *t, uint32_t n)
{
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i < n)
        t[i] = s[i];
}

bool bad(const void *p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// The streaming launcher's reservation, for the same unit count.
unsigned cap_lds(uint64_t vecs, unsigned lds) { return vecs >= glu::kCapMinUnits ? lds : 0u; }

}  // namespace

extern "C" {

GLU_REF_API int glu_ref_fwd_mix(const void *a, const void *b, void *y, uint64_t bytes, hipStream_t stream)
{
    if (bad(a) || bad(b) || bad(y) || (bytes & 15u) != 0)
        return -1;
    constexpr int B = GLU_BLOCK_FWD;
    const uint64_t n = bytes / 16;
    const unsigned lds = cap_lds(n, glu::kCapLdsFwd);
    for (uint64_t v0 = 0; v0 < n; v0 += kMaxVecs) {
        const uint32_t m = uint32_t(n - v0 < kMaxVecs ? n - v0 : kMaxVecs);
        hipLaunchKernelGGL(fwd_mix_kernel<B>, dim3((m + B - 1) / B), dim3(B), lds, stream,
                           static_cast<const u32x4 *>(a) + v0, static_cast<const u32x4 *>(b) + v0,
                           static_cast<u32x4 *>(y) + v0, m);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return int(e);
    }
    return 0;
}

GLU_REF_API int glu_ref_bwd_mix(const void *a, const void *b, const void *dy, void *da, void *db, uint64_t bytes,
                                hipStream_t stream)
{
    if (bad(a) || bad(b) || bad(dy) || bad(da) || bad(db) || (bytes & 15u) != 0)
        return -1;
    const uint64_t n = bytes / 16;
    const unsigned lds = cap_lds(n, glu::kCapLdsBwd);
    // the streaming launcher's block size for the same unit count
    const bool small = n < glu::kCapMinUnits;
    for (uint64_t v0 = 0; v0 < n; v0 += kMaxVecs) {
        const uint32_t m = uint32_t(n - v0 < kMaxVecs ? n - v0 : kMaxVecs);
        const u32x4 *pa = static_cast<const u32x4 *>(a) + v0, *pb = static_cast<const u32x4 *>(b) + v0,
                    *pd = static_cast<const u32x4 *>(dy) + v0;
        u32x4 *pda = static_cast<u32x4 *>(da) + v0, *pdb = static_cast<u32x4 *>(db) + v0;
        if (small) {
            constexpr int B = GLU_BLOCK_BWD_SMALL;
            hipLaunchKernelGGL(bwd_mix_kernel<B>, dim3((m + B - 1) / B), dim3(B), lds, stream, pa, pb, pd, pda, pdb, m);
        } else {
            constexpr int B = GLU_BLOCK_BWD;
            hipLaunchKernelGGL(bwd_mix_kernel<B>, dim3((m + B - 1) / B), dim3(B), lds, stream, pa, pb, pd, pda, pdb, m);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return int(e);
    }
    return 0;
}

GLU_REF_API int glu_ref_rms_mix(const void *x, const void *r, void *h, void *y, uint64_t bytes, hipStream_t stream)
{
    if (bad(x) || bad(r) || bad(h) || bad(y) || (bytes & 15u) != 0)
        return -1;
    const uint64_t n = bytes / 16;
    for (uint64_t v0 = 0; v0 < n; v0 += kMaxVecs) {
        const uint32_t m = uint32_t(n - v0 < kMaxVecs ? n - v0 : kMaxVecs);
        hipLaunchKernelGGL(rms_mix_kernel, dim3((m + 63) / 64), dim3(64), glu::kCapLdsFwd, stream,
                           static_cast<const u32x4 *>(x) + v0, static_cast<const u32x4 *>(r) + v0,
                           static_cast<u32x4 *>(h) + v0, static_cast<u32x4 *>(y) + v0, m);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return int(e);
    }
    return 0;
}

GLU_REF_API int glu_ref_tile_bwd_mix(const void *a, const void *b, const void *dyT, void *da, void *db, int64_t rows,
                                     int64_t cols, hipStream_t stream)
{
    if (bad(a) || bad(b) || bad(dyT) || bad(da) || bad(db) || !tile_shape_ok(rows, cols))
        return -1;
    const uint32_t tr = uint32_t(rows / kT), tcn = uint32_t(cols / kT);
    hipLaunchKernelGGL(tile_bwd_mix_kernel, dim3(tr * tcn), dim3(256), kTileMixDynLds, stream,
                       static_cast<const uint16_t *>(a), static_cast<const uint16_t *>(b),
                       static_cast<const uint16_t *>(dyT), static_cast<uint16_t *>(da), static_cast<uint16_t *>(db), rows,
                       cols, tr, tcn);
    return int(hipGetLastError());
}

GLU_REF_API int glu_ref_tile_fwd_mix(const void *a, const void *b, void *yT, int64_t rows, int64_t cols,
                                     hipStream_t stream)
{
    if (bad(a) || bad(b) || bad(yT) || !tile_shape_ok(rows, cols))
        return -1;
    const uint32_t tr = uint32_t(rows / kT), tcn = uint32_t(cols / kT);
    hipLaunchKernelGGL(tile_fwd_mix_kernel, dim3(tr * tcn), dim3(256), kTileMixDynLds, stream,
                       static_cast<const uint16_t *>(a), static_cast<const uint16_t *>(b), static_cast<uint16_t *>(yT),
                       rows, cols, tr, tcn);
    return int(hipGetLastError());
}

GLU_REF_API int glu_ref_copy(const void *src, void *dst, uint64_t bytes, hipStream_t stream)
{
    if (bad(src) || bad(dst) || (bytes & 15u) != 0)
        return -1;
    const uint64_t n = bytes / 16;
    for (uint64_t v0 = 0; v0 < n; v0 += kMaxVecs) {
        const uint32_t m = uint32_t(n - v0 < kMaxVecs ? n - v0 : kMaxVecs);
        hipLaunchKernelGGL(copy_kernel, dim3((m + 255) / 256), dim3(256), 0, stream,
                           static_cast<const u32x4 *>(src) + v0, static_cast<u32x4 *>(dst) + v0, m);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return int(e);
    }
    return 0;
}

}  // extern "C"
