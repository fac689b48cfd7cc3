// gemm_kernels.hip -- gfx950 MFMA kernel for the gate/up projection with the
// gated activation fused into its epilogue:
//   g = x @ wg^T,  u = x @ wu^T,  h = act(g) * u
// ("Fused Kernels", section 4: gate and up tiles are accumulated and the
// activation is applied in registers; "Write a Triton SiLU-Mul (SwiGLU)
// Kernel", Do not use this when / Performance requirements: fusing the
// activation into the matmul epilogue saves the round trip of g and u
// through HBM).
//
// This is a dense contraction, so it runs on the matrix cores:
//  - for many tokens, a workgroup of 512 threads (8 waves, 4 x 2; two per
//    SIMD, so one wave's LDS and barrier waits are covered by the other's
//    MFMAs) owns 256 rows of x and 128 columns of h, i.e. 128 gate and 128 up
//    rows of the weights; each wave holds a 64 x 64 block of g and the same
//    block of u in 8 fp32 accumulators of v_mfma_f32_32x32x16_{bf16,f16};
//  - for few tokens (at most 256), where streaming the weights bounds the
//    kernel, a workgroup of 256 threads (4 waves, 2 x 2) owns 128 rows of x
//    and 64 columns of h, so N / 64 workgroups spread the weights over every
//    CU; each wave holds a 64 x 32 block of g and of u.  Both tiles sum k in
//    the same order, so their results are bit-identical;
//  - both operands are k-contiguous (x rows, weight rows), so every MFMA
//    fragment is one 16-byte LDS read;
//  - k advances 64 at a time through two LDS stages of 64 KiB; the next
//    stage is fetched with direct global-to-LDS loads (no registers, no LDS
//    write instructions) while the current stage's MFMAs run; stage rows are
//    128 bytes with XOR-swizzled 16-byte chunks so fragment reads spread
//    over the banks; the MFMA fragments of the next 16-deep k step are read
//    while the current step's MFMAs issue, and the one barrier per stage sits
//    before the stage's last MFMAs, which cover it and the first fragment
//    reads of the next stage;
//  - g and u of one element sit in the same lane and register slot, so the
//    epilogue act(g) * u is lane-local; h is rounded once to the storage type,
//    staged through LDS and written in whole cache lines.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "glu_act.h"
#include "glu_internal.h"
#include "gemm_internal.h"

namespace glu {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// v_mfma_f32_32x32x16: 32 x 32 blocks, 16 deep, 16 accumulator registers.
// (A 16 x 16 x 32 variant of this tiling needs twice the fragment registers
// and spills.)
constexpr int MF = 32, KD = 16;
typedef f32x16 AccT;
constexpr int ACC_E = MF * MF / 64;   // accumulator registers per lane

template <typename E> struct MfmaOp;
template <> struct MfmaOp<__bf16> {
    __device__ static AccT run(u32x4 a, u32x4 b, AccT c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
};
template <> struct MfmaOp<_Float16> {
    __device__ static AccT run(u32x4 a, u32x4 b, AccT c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    }
};

// Tile configurations.  Wave w of WAVES works on tokens [TPW (w / WN), +TPW)
// and features [FPW (w % WN), +FPW) of the workgroup tile, FPW = BN / WN, in
// (TPW / 32) x (FPW / 32) blocks of g and as many of u.  LDS_BYTES of LDS
// hold NST stages of (BM + 2 BN) rows x BK.  OCC: workgroups per CU the
// launch bounds allow.
template <int BM_, int BN_, int WAVES_, int WN_, int LDS_BYTES_, int OCC_> struct GemmCfg {
    static constexpr int BM = BM_, BN = BN_, WAVES = WAVES_, WN = WN_, LDS_BYTES = LDS_BYTES_, OCC = OCC_;
};
#ifndef GLU_GEMM_WAVES
#define GLU_GEMM_WAVES 8   // 4 (one wave per SIMD, 128 x 64 per wave) measured 8 % slower
#endif
// Small tiles: three 32 KiB stages.  Swept at 4096 -> 14336 bf16, one wave
// per SIMD: 64 KiB (two stages) 66-68 us at M <= 128, 96 KiB 50-55, 128 KiB
// the same as 96; at M = 192-256 two stages won (77-85 against 82-88 us),
// where both lose to the unfused path anyway.
#ifndef GLU_GEMM_SMALL_LDS
#define GLU_GEMM_SMALL_LDS (96 * 1024)
#endif
#ifndef GLU_GEMM_SMALL_OCC
#define GLU_GEMM_SMALL_OCC 1
#endif
using CfgLarge = GemmCfg<256, 128, GLU_GEMM_WAVES, 2, 128 * 1024, 1>;
using CfgSmall = GemmCfg<128, 64, 4, 2, GLU_GEMM_SMALL_LDS, GLU_GEMM_SMALL_OCC>;

constexpr int BK = kGemmBK;
constexpr int ROW_BYTES = BK * 2;               // one row of a stage
constexpr int CPR = BK / 8;                     // 16-byte chunks per row
constexpr int RPI = 1024 / ROW_BYTES;           // rows per wave load instruction (1 KiB)
constexpr int KSTEPS = BK / KD;                 // MFMA k steps per stage
static_assert(KSTEPS % 2 == 0, "fragment double buffer alternates within a stage");

// Chunk c of stage row r sits at position c ^ swz(r) of the row.  The 16
// lanes one LDS cycle serves read 16 consecutive rows at one logical chunk;
// rows 256 bytes apart share banks, so they get distinct positions.
__device__ inline int swz(int r) { return (r / (256 / ROW_BYTES)) % CPR; }

typedef __attribute__((address_space(3))) void lds_t;
typedef const __attribute__((address_space(1))) void gbl_t;

// Scheduling hints for the compiler's machine scheduler (instruction-class
// masks of __builtin_amdgcn_sched_group_barrier).
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100;

// s_waitcnt immediates: wait until at most n of this wave's vector-memory
// loads are outstanding (n < 64), LDS and export counters untouched.
template <int n> constexpr int vm_wait() { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Workgroup barrier without a memory fence: the caller has already waited for
// its own LDS writes (the counters above); the empty asm keeps the compiler
// from moving memory accesses across it.
__device__ inline void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <typename E, int KIND, typename C>
__global__ void __launch_bounds__(64 * C::WAVES, C::OCC) gemm_glu_kernel(const GemmArgs p)
{
    constexpr int BM = C::BM, BN = C::BN, WAVES = C::WAVES, WN = C::WN, WM = WAVES / WN;
    constexpr int ROWS = BM + 2 * BN;               // x rows, then gate rows, then up rows
    constexpr int STAGE_BYTES = ROWS * ROW_BYTES;
    constexpr int NST = C::LDS_BYTES / STAGE_BYTES; // LDS stages, all in flight
    constexpr int THREADS = 64 * WAVES;
    constexpr int RPW = ROWS / WAVES;               // stage rows each wave loads
    constexpr int TPW = BM / WM;                    // tokens (x rows) each wave computes
    constexpr int FPW = BN / WN;                    // features (of g and of u) each wave computes
    constexpr int LOADS = RPW / RPI;                // load instructions per wave per stage
    constexpr int FX = TPW / MF;                    // x (token) fragments per wave
    constexpr int FW = FPW / MF;                    // gate (and up) fragments per wave
    constexpr int NREAD = FX + 2 * FW;              // fragment reads per k step
    constexpr int NMFMA = FX * 2 * FW;              // MFMAs per k step
    static_assert(NST >= 2 && NST <= 4, "two to four stages");
    static_assert(ROWS % WAVES == 0 && RPW % RPI == 0 && BM % RPW == 0 && BN % RPW == 0,
                  "each wave loads whole instructions of one operand");
    static_assert(TPW % MF == 0 && FPW % MF == 0 && NMFMA >= NREAD, "whole fragments per wave");
    __shared__ u32x4 lds_v[NST * STAGE_BYTES / 16];
    char *lds = reinterpret_cast<char *>(lds_v);

    const uint32_t nt = p.tiles_m * p.tiles_n;
    const TileCoord tc = grouped_coord(xcd_remap(blockIdx.x, nt), p.tiles_m, p.tiles_n, kGemmGroup);
    const int64_t m0 = int64_t(tc.r) * BM, n0 = int64_t(tc.c) * BN;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w / WN, wn = w % WN;

    // Loads: wave w fills stage rows [RPW w, RPW w + RPW): x rows, then
    // gate rows, then up rows.  Instruction j covers rows
    // RPW w + RPI j + lane / CPR; lane puts logical chunk
    // (lane % CPR) ^ swz(row) at position lane % CPR, i.e. at LDS byte
    // row * ROW_BYTES + 16 * (lane % CPR): one contiguous KiB per wave
    // instruction, the layout the direct-to-LDS load writes.  Rows past M or
    // N are read from a valid row (clamped); their results are never stored.
    // The wave index is uniform: keep everything the load addresses need in
    // scalar registers, plus one 32-bit byte offset per lane and instruction
    // from the tile's first row (row strides are below 2^24 elements, so the
    // offsets fit).
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const char *gbase;
    int64_t gld, gfirst, glimit;
    const int r0 = RPW * wu;   // first stage row this wave loads
    if (r0 < BM) {
        gbase = static_cast<const char *>(p.x);
        gld = p.ldx;
        gfirst = m0 + r0;
        glimit = p.M;
    } else {
        const bool gate = r0 < BM + BN;
        gbase = static_cast<const char *>(gate ? p.wg : p.wu);
        gld = gate ? p.ldwg : p.ldwu;
        gfirst = n0 + (gate ? r0 - BM : r0 - BM - BN);
        glimit = p.N;
    }
    const int64_t fc = gfirst < glimit ? gfirst : glimit - 1;
    const char *tbase = gbase + fc * gld * 2;
    const int lrow = lane / CPR, lpos = lane % CPR;
    uint32_t goff[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const int r = r0 + RPI * j + lrow;
        int64_t row = gfirst + RPI * j + lrow;
        row = row < glimit ? row : glimit - 1;
        goff[j] = uint32_t(((row - fc) * gld + 8 * (lpos ^ swz(r))) * 2);
    }
    auto issue_direct = [&](int buf, int k0, int j) {
        __builtin_amdgcn_global_load_lds((gbl_t *)(tbase + int64_t(k0) * 2 + uint64_t(goff[j])),
                                         (lds_t *)(lds + buf * STAGE_BYTES + (r0 + RPI * j) * ROW_BYTES), 16,
                                         0, 0);
    };
    // The last stage may be partial: zero past K, through registers (the
    // waits before the next barrier cover its LDS writes).
    auto issue_partial = [&](int buf, int k0) {
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int r = r0 + RPI * j + lrow;
            const int kc = 8 * (lpos ^ swz(r));
            const u32x4 v = k0 + kc < p.K ? *reinterpret_cast<const u32x4 *>(tbase + int64_t(k0) * 2 + uint64_t(goff[j]))
                                          : u32x4{0, 0, 0, 0};
            *reinterpret_cast<u32x4 *>(lds + buf * STAGE_BYTES + r * ROW_BYTES + 16 * lpos) = v;
        }
    };

    AccT accg[FX][FW], accu[FX][FW];
#pragma unroll
    for (int i = 0; i < FX; ++i)
#pragma unroll
        for (int j = 0; j < FW; ++j) {
            accg[i][j] = AccT{0};
            accu[i][j] = AccT{0};
        }

    // Fragment reads: lane reads row (lane % MF) of each fragment at logical
    // chunk KD/8 * ks + lane / MF; row r, chunk c -> LDS byte
    // r*ROW_BYTES + 16*(c ^ swz(r)).
    const int kq = lane / MF;
    const int ra = wm * TPW + (lane % MF), rg = BM + wn * FPW + (lane % MF), ru = BM + BN + wn * FPW + (lane % MF);
    struct Frags {
        u32x4 a[FX], g[FW], u[FW];
    };
    auto frag = [&](const char *st, int r, int ks) -> u32x4 {
        return *reinterpret_cast<const u32x4 *>(st + r * ROW_BYTES + 16 * (((KD / 8) * ks + kq) ^ swz(r)));
    };
    auto read = [&](const char *st, int ks, Frags &f) {
#pragma unroll
        for (int i = 0; i < FX; ++i)
            f.a[i] = frag(st, ra + MF * i, ks);
#pragma unroll
        for (int j = 0; j < FW; ++j) {
            f.g[j] = frag(st, rg + MF * j, ks);
            f.u[j] = frag(st, ru + MF * j, ks);
        }
    };
    auto mfmas = [&](const Frags &f) {
#pragma unroll
        for (int i = 0; i < FX; ++i)
#pragma unroll
            for (int j = 0; j < FW; ++j) {
                accg[i][j] = MfmaOp<E>::run(f.g[j], f.a[i], accg[i][j]);
                accu[i][j] = MfmaOp<E>::run(f.u[j], f.a[i], accu[i][j]);
            }
    };
    // Wait until at most `ahead` later stages of this wave's loads are in
    // flight and this wave's LDS reads are done, then barrier: the next stage
    // is in LDS, and no wave still reads the buffer about to be refilled.
    auto wait_stage = [&](int ahead) {
        if (ahead >= 3)   // at most NST - 1 <= 3
            __builtin_amdgcn_s_waitcnt(vm_wait<3 * LOADS>());
        else if (ahead == 2)
            __builtin_amdgcn_s_waitcnt(vm_wait<2 * LOADS>());
        else if (ahead == 1)
            __builtin_amdgcn_s_waitcnt(vm_wait<LOADS>());
        else
            __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_waitcnt(vm_wait<63>() & ~(15 << 8));   // LDS writes of the partial stage
        lds_barrier();
    };

    const int KT = (p.K + BK - 1) / BK, KF = p.K / BK;   // stages, full stages
    // Steps 0 .. KSTEPS-2 of a stage: the fragments of step ks + 1 are read
    // while step ks's MFMAs issue.
    auto steps = [&](const char *st, Frags *f) {
#pragma unroll
        for (int ks = 0; ks + 1 < KSTEPS; ++ks) {
            read(st, ks + 1, f[(ks + 1) & 1]);
            mfmas(f[ks & 1]);
#pragma unroll
            for (int q = 0; q < NREAD; ++q) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
            }
            if constexpr (NMFMA > NREAD)
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, NMFMA - NREAD, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Prologue: every buffer, then stage 0's first fragments.  A buffer is
    // refilled only once its own stage has been read, so all NST stages are
    // in flight together.
#pragma unroll
    for (int s = 0; s < NST; ++s) {
        if (s < KF)
            for (int j = 0; j < LOADS; ++j)
                issue_direct(s, s * BK, j);
        else if (s < KT)
            issue_partial(s, s * BK);
    }
    Frags f[2];
    {
        const int ahead = KT - 1 < NST - 1 ? KT - 1 : NST - 1;
        wait_stage(ahead);
        read(lds, 0, f[0]);
    }
    // The barrier of stage kt + 1 sits inside stage kt's last step, between
    // its fragment reads (done: the fragments are in registers) and its MFMAs,
    // which then cover the barrier, the loads into the buffer just freed
    // (stage kt's own) and the fragment reads of stage kt + 1's first step.
    int kt = 0;
    for (; kt + NST < KF; ++kt) {
        steps(lds + (kt % NST) * STAGE_BYTES, f);
        wait_stage(NST - 2);
#pragma unroll
        for (int j = 0; j < LOADS; ++j)
            issue_direct(kt % NST, (kt + NST) * BK, j);
        read(lds + ((kt + 1) % NST) * STAGE_BYTES, 0, f[0]);
        mfmas(f[1]);
#pragma unroll
        for (int q = 0; q < NREAD; ++q) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, (LOADS + NREAD - 1) / NREAD, 0);
        }
        if constexpr (NMFMA > NREAD)
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, NMFMA - NREAD, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (; kt < KT; ++kt) {
        steps(lds + (kt % NST) * STAGE_BYTES, f);
        if (kt + 1 < KT) {
            const int ahead = KT - 2 - kt < NST - 2 ? KT - 2 - kt : NST - 2;
            wait_stage(ahead);
            const int s = kt + NST;
            if (s < KF)
                for (int j = 0; j < LOADS; ++j)
                    issue_direct(kt % NST, s * BK, j);
            else if (s < KT)
                issue_partial(kt % NST, s * BK);
            read(lds + ((kt + 1) % NST) * STAGE_BYTES, 0, f[0]);
        }
        mfmas(f[1]);
        __builtin_amdgcn_sched_barrier(0);
    }
    lds_barrier();

    // Epilogue.  The MFMAs take the weight rows as their first operand, so
    // each 32 x 32 block is g^T: lane holds token row m = lane % 32 of the
    // block and, for e < 16, feature column 8*(e/4) + 4*(lane/32) + e%4.
    // Each output tile (h, then g and u when asked for) is staged through
    // LDS, now free, as 256 token rows of 128 features (rows padded to 272
    // bytes), and leaves in 16-byte non-temporal stores, 16 lanes per
    // 256-byte token row: whole cache lines, where direct 8-byte stores from
    // the MFMA layout would leave partial lines.
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    typedef E ex4 __attribute__((ext_vector_type(4)));
    constexpr int OPITCH = BN * 2 + 16;   // bytes per staged token row
    constexpr int OCPR = BN / 8;          // 16-byte output chunks per token row
    static_assert(BM * OPITCH <= NST * STAGE_BYTES, "output tile fits the stage buffers");
    static_assert((BM * OCPR) % THREADS == 0, "whole output chunks per thread");
    auto put = [&](E *dst, int64_t ld, auto value) {
        // this wave's values -> LDS
#pragma unroll
        for (int i = 0; i < FX; ++i)
#pragma unroll
            for (int j = 0; j < FW; ++j)
#pragma unroll
                for (int q = 0; q < ACC_E / 4; ++q) {
                    ex4 v4;
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        v4[t] = static_cast<E>(value(i, j, 4 * q + t));
                    const int row = wm * TPW + i * MF + (lane % MF);
                    const int col = wn * FPW + j * MF + q * 8 + (lane >> 5) * 4;
                    *reinterpret_cast<u32x2 *>(lds + row * OPITCH + col * 2) = __builtin_bit_cast(u32x2, v4);
                }
        __builtin_amdgcn_s_waitcnt(0);
        lds_barrier();
        // LDS -> memory: chunk c covers token row c / OCPR, features 8 (c % OCPR) .. + 7
#pragma unroll
        for (int k = 0; k < BM * OCPR / THREADS; ++k) {
            const int c = tid + THREADS * k, row = c / OCPR, col = (c % OCPR) * 8;
            const int64_t m = m0 + row, n = n0 + col;
            if (m >= p.M || n >= p.N)
                continue;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(lds + row * OPITCH + col * 2);
            E *out = dst + m * ld + n;
            if (n + 8 <= p.N && (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
                // streaming store: the L2 keeps the x and weight rows the
                // other tiles still read (725 against 739 us at 4096 x 4096
                // -> 14336)
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(out));
            } else {
                const E *e = reinterpret_cast<const E *>(&v);
                for (int t = 0; t < 8 && n + t < p.N; ++t)
                    out[t] = e[t];
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        lds_barrier();   // the tile is out of LDS before the next one goes in
    };
    put(static_cast<E *>(p.h), p.ldh,
        [&](int i, int j, int e) { return act<KIND, float>(accg[i][j][e]) * accu[i][j][e]; });
    if (p.gu) {
        E *gu = static_cast<E *>(p.gu);
        put(gu, p.ldgu, [&](int i, int j, int e) { return accg[i][j][e]; });
        put(gu + p.N, p.ldgu, [&](int i, int j, int e) { return accu[i][j][e]; });
    }
}

typedef void (*GemmFn)(const GemmArgs);

template <typename E, typename C> GemmFn pick_gemm(int kind)
{
    switch (kind) {
    case SILU: return &gemm_glu_kernel<E, SILU, C>;
    case GELU_ERF: return &gemm_glu_kernel<E, GELU_ERF, C>;
    case GELU_TANH: return &gemm_glu_kernel<E, GELU_TANH, C>;
    default: return &gemm_glu_kernel<E, RELU, C>;
    }
}

template <typename C> hipError_t launch_cfg(int dtype, int kind, const GemmArgs &args, hipStream_t stream)
{
    static_assert(C::BM == kGemmTiles[std::is_same<C, CfgSmall>::value ? kGemmSmall : kGemmLarge].bm &&
                      C::BN == kGemmTiles[std::is_same<C, CfgSmall>::value ? kGemmSmall : kGemmLarge].bn,
                  "the host plans tiles with the same shape");
    GemmFn fn = dtype == F16 ? pick_gemm<_Float16, C>(kind) : pick_gemm<__bf16, C>(kind);
    GemmArgs copy = args;
    void *kargs[] = {&copy};
    return hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3(args.tiles_m * args.tiles_n), dim3(64 * C::WAVES),
                           kargs, 0, stream);
}

}  // namespace

hipError_t launch_gemm_glu(int dtype, int kind, const GemmArgs &args, hipStream_t stream)
{
    return args.config == kGemmSmall ? launch_cfg<CfgSmall>(dtype, kind, args, stream)
                                     : launch_cfg<CfgLarge>(dtype, kind, args, stream);
}

}  // namespace glu
