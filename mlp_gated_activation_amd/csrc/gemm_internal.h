// gemm_internal.h -- the launch plan passed from the host API (glu_api.cpp)
// to the gate/up projection kernels (gemm_kernels.hip).  Not part of the
// public ABI.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace glu {

// ---------------------------------------------------------------------------
// Gate/up projection with the activation in the epilogue (gemm_kernels.hip).
// Workgroup tile: bm rows of x by bn columns of h, i.e. bn gate rows and bn
// up rows of the weights, kGemmBK deep per stage.  Two tile configurations:
//  - kGemmLarge, 256 x 128 (8 waves), for many tokens, where the MFMAs bound
//    the kernel;
//  - kGemmSmall, 128 x 64 (4 waves), for few tokens (M <= kGemmSmallMaxM),
//    where streaming the weights from HBM bounds it: 256 x 128 tiles give
//    N / 128 workgroups (112 at N = 14336), fewer than the 256 CUs, and the
//    weights then stream at less than half the bandwidth.
// ---------------------------------------------------------------------------
#ifndef GLU_GEMM_BK
#define GLU_GEMM_BK 64
#endif
constexpr int kGemmBK = GLU_GEMM_BK;
#ifndef GLU_GEMM_GROUP
#define GLU_GEMM_GROUP 4
#endif
constexpr uint32_t kGemmGroup = GLU_GEMM_GROUP;   // row tiles per group of the launch order

enum GemmConfig { kGemmLarge = 0, kGemmSmall = 1 };
struct GemmTile {
    int bm, bn;
};
constexpr GemmTile kGemmTiles[2] = {{256, 128}, {128, 64}};
#ifndef GLU_GEMM_SMALL_MAX_M
#define GLU_GEMM_SMALL_MAX_M 256
#endif
constexpr int64_t kGemmSmallMaxM = GLU_GEMM_SMALL_MAX_M;
inline int gemm_config(int64_t M) { return M <= kGemmSmallMaxM ? kGemmSmall : kGemmLarge; }

struct GemmArgs {
    const void *x, *wg, *wu;  // x: M x K, wg / wu: N x K ([out][in]), 16-byte aligned rows
    void *h;                  // M x N
    void *gu;                 // optional: g at gu[m][n], u at gu[m][N + n] (or NULL)
    int64_t ldx, ldwg, ldwu, ldh, ldgu;
    int32_t M, N, K;
    uint32_t tiles_m, tiles_n;  // of the configuration's tile
    int32_t config;             // GemmConfig
};
// Largest workgroup count of one GEMM launch (grid * 256 below 2^32).
constexpr uint32_t kMaxGemmTiles = 1u << 24;
// Input row strides stay below this (elements): a wave addresses its 64
// stage rows of an operand with 32-bit byte offsets.
constexpr int64_t kGemmMaxLd = int64_t(1) << 24;

hipError_t launch_gemm_glu(int dtype, int kind, const GemmArgs &args, hipStream_t stream);

}  // namespace glu
