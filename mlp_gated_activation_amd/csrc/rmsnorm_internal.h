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
    int rpb;   // rows per workgroup: > 1 selects the pipelined multi-row kernel
};
// Shapes measured on MI355X (bf16, 4096 rows): one 64-lane wave per row up
// to 8 vectors per lane (H <= 4096), then 4 vectors per lane with the block
// grown to the row (8192: 256 threads, 16384: 512), 8 per lane only past
// 32768.  Each entry: smallest row capacity first.  Rows per workgroup, from
// a sweep of 1, 2, 4 and 8 (bf16, 4096 rows, H = 2048 .. 16384): 4 for the
// 8192-wide shape (5930 against 5758 GB/s at 4096 x 8192); 1 elsewhere,
// where fewer, longer-lived workgroups lost (4096 x 4096: 5613 against
// 5195 at 2 rows and 3496 at 4).  GLU_RMS_RPB > 0 overrides it for sweeps.
#ifndef GLU_RMS_TABLE
#define GLU_RMS_TABLE 3
#endif
#ifndef GLU_RMS_RPB
#define GLU_RMS_RPB 0
#endif
#if GLU_RMS_TABLE == 0
constexpr RmsShape kRmsShapes[] = {{64, 1, 1}, {128, 1, 1}, {256, 1, 1}, {256, 2, 1}, {256, 4, 1}, {256, 8, 1}, {512, 8, 1}, {1024, 8, 1}};
#elif GLU_RMS_TABLE == 1
constexpr RmsShape kRmsShapes[] = {{64, 1, 1}, {64, 2, 1}, {64, 4, 1}, {64, 8, 1}, {128, 8, 1}, {256, 8, 1}, {512, 8, 1}, {1024, 8, 1}};
#elif GLU_RMS_TABLE == 2
constexpr RmsShape kRmsShapes[] = {{64, 1, 1}, {64, 2, 1}, {64, 4, 1}, {128, 4, 1}, {256, 4, 1}, {512, 4, 1}, {512, 8, 1}, {1024, 8, 1}};
#else
constexpr RmsShape kRmsShapes[] = {{64, 1, 1}, {64, 2, 1}, {64, 4, 1}, {64, 8, 1}, {256, 4, 4}, {512, 4, 1}, {1024, 4, 1}, {1024, 8, 1}};
#endif
constexpr int kRmsLoopBlock = 1024;

// Picks the smallest single-pass shape holding `hidden` elements with `ve`
// elements per vector; {kRmsLoopBlock, 0, 1} if none does.
inline RmsShape rms_shape(int64_t hidden, int ve)
{
    for (const RmsShape &s : kRmsShapes)
        if (int64_t(s.block) * s.vpt * ve >= hidden)
            return RmsShape{s.block, s.vpt, GLU_RMS_RPB > 0 ? GLU_RMS_RPB : s.rpb};
    return RmsShape{kRmsLoopBlock, 0, 1};
}

hipError_t launch_add_rmsnorm(int dtype, bool vec, RmsShape shape, uint32_t rows, const RmsArgs &args,
                              hipStream_t stream);

}  // namespace glu
