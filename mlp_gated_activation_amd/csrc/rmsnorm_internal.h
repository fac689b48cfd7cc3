// rmsnorm_internal.h -- the launch plan passed from the host API
// (glu_api.cpp) to the fused residual add + RMSNorm kernels
// (rmsnorm_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace glu {

// Fused residual add + RMSNorm forward: one workgroup per row.
struct RmsArgs {
    const void *x;
    const void *res;
    const void *gamma;
    void *h;
    void *y;
    float *rstd;     // may be null
    int64_t ldx, ldr, ldh, ldy;
    uint32_t hidden; // elements per row (<= 2^31)
    float eps;
};

// Row capacities of the single-pass (registers) kernels: block threads x
// vectors per thread.  Rows wider than the largest use the two-pass kernel,
// which recomputes h = x + residual and therefore needs x, residual intact.
struct RmsShape {
    int block;
    int vpt;   // 0: two-pass loop
};
// Shapes measured on MI355X (bf16, 4096 rows): one 64-lane wave per row up
// to 8 vectors per lane (H <= 4096), then 4 vectors per lane with the block
// grown to the row (8192: 256 threads, 16384: 512), 8 per lane only past
// 32768.  Each entry: smallest row capacity first.
#ifndef GLU_RMS_TABLE
#define GLU_RMS_TABLE 3
#endif
#if GLU_RMS_TABLE == 0
constexpr RmsShape kRmsShapes[] = {{64, 1}, {128, 1}, {256, 1}, {256, 2}, {256, 4}, {256, 8}, {512, 8}, {1024, 8}};
#elif GLU_RMS_TABLE == 1
constexpr RmsShape kRmsShapes[] = {{64, 1}, {64, 2}, {64, 4}, {64, 8}, {128, 8}, {256, 8}, {512, 8}, {1024, 8}};
#elif GLU_RMS_TABLE == 2
constexpr RmsShape kRmsShapes[] = {{64, 1}, {64, 2}, {64, 4}, {128, 4}, {256, 4}, {512, 4}, {512, 8}, {1024, 8}};
#else
constexpr RmsShape kRmsShapes[] = {{64, 1}, {64, 2}, {64, 4}, {64, 8}, {256, 4}, {512, 4}, {1024, 4}, {1024, 8}};
#endif
constexpr int kRmsLoopBlock = 1024;

// Picks the smallest single-pass shape holding `hidden` elements with `ve`
// elements per vector; {kRmsLoopBlock, 0} if none does.
inline RmsShape rms_shape(int64_t hidden, int ve)
{
    for (const RmsShape &s : kRmsShapes)
        if (int64_t(s.block) * s.vpt * ve >= hidden)
            return s;
    return RmsShape{kRmsLoopBlock, 0};
}

hipError_t launch_add_rmsnorm(int dtype, bool vec, RmsShape shape, uint32_t rows, const RmsArgs &args,
                              hipStream_t stream);

}  // namespace glu
