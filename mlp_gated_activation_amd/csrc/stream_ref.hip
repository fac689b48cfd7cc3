// stream_ref.hip -- data-movement reference kernels (include/glu_ref.h).
//
// Measurement infrastructure, not part of the method: the mix kernels move
// the bytes of one streaming gated-activation launch with the same
// per-thread access (one 16-byte non-temporal vector per stream), the same
// workgroup size and the same LDS reservation that caps resident workgroups
// per CU, and replace the arithmetic by an XOR; the RMSNorm mix moves the
// fused add + RMSNorm forward's bytes as a flat stream.  Built into its own
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
    constexpr int B = GLU_BLOCK_BWD;
    const uint64_t n = bytes / 16;
    const unsigned lds = cap_lds(n, glu::kCapLdsBwd);
    for (uint64_t v0 = 0; v0 < n; v0 += kMaxVecs) {
        const uint32_t m = uint32_t(n - v0 < kMaxVecs ? n - v0 : kMaxVecs);
        hipLaunchKernelGGL(bwd_mix_kernel<B>, dim3((m + B - 1) / B), dim3(B), lds, stream,
                           static_cast<const u32x4 *>(a) + v0, static_cast<const u32x4 *>(b) + v0,
                           static_cast<const u32x4 *>(dy) + v0, static_cast<u32x4 *>(da) + v0,
                           static_cast<u32x4 *>(db) + v0, m);
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
