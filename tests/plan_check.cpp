// Host-only check of the launch planner in glu_api.cpp.
//
// glu::launch is replaced by a stub that records each launch's Args instead
// of enqueuing a kernel.  For a given call the program then verifies, for
// every recorded launch, the kernel's own 32-bit index arithmetic at the
// boundary units (first/last unit of a launch, of rows, around 2^k), and that
// the launches tile the rows x cols problem exactly once.
//
// usage: plan_check <fwd|bwd> <layout> <dtype> <rows> <cols> <ld_in> <ld_out> <misalign>
//        plan_check inplace      (exact in-place aliasing is accepted)
// prints "ok <launches>" or "FAIL <reason>".
#include "glu.h"
#include "glu_internal.h"
#include "gemm_internal.h"
#include "rmsnorm_internal.h"

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <vector>

namespace glu {
static std::vector<Args> g_launches;
static std::vector<bool> g_vec;
hipError_t launch(int, int, bool, bool vec, const Args &args, hipStream_t)
{
    g_launches.push_back(args);
    g_vec.push_back(vec);
    return hipSuccess;
}
hipError_t launch_gemm_glu(int, int, const GemmArgs &, hipStream_t)
{
    return hipSuccess;   // not exercised here
}
hipError_t launch_add_rmsnorm(int, bool, RmsShape, uint32_t, const RmsArgs &, hipStream_t)
{
    return hipSuccess;   // not exercised here
}
hipError_t launch_tiles(int, int, bool, const TileArgs &, uint32_t, hipStream_t)
{
    return hipSuccess;   // not exercised here
}
}  // namespace glu

static int fail(const char *why, long long a = 0, long long b = 0)
{
    std::printf("FAIL %s %lld %lld\n", why, a, b);
    return 1;
}

// In-place calls the boundary must accept: a forward whose y := b is exactly
// a (so a == b), and the [gate | up] forward whose y := b is x's second half.
static int accepted_inplace()
{
    const uintptr_t A = uintptr_t(1) << 44;
    glu_status st = glu_fwd(GLU_SILU, GLU_SEPARATE, GLU_BF16, 4, 64, (void *)A, 64, (void *)A, 64, nullptr, 64,
                            1, nullptr);
    if (st != GLU_OK || glu::g_launches.size() != 1 || glu::g_launches[0].out0 != (void *)A)
        return fail("a == b in place", st);
    st = glu_fwd(GLU_SILU, GLU_GATE_UP, GLU_BF16, 4, 64, (void *)A, 128, nullptr, 0, nullptr, 0, 1, nullptr);
    if (st != GLU_OK || glu::g_launches.size() != 2 || glu::g_launches[1].out0 != (void *)(A + 128))
        return fail("gate_up in place", st);
    std::printf("ok %zu\n", glu::g_launches.size());
    return 0;
}

int main(int argc, char **argv)
{
    if (argc == 2 && std::strcmp(argv[1], "inplace") == 0)
        return accepted_inplace();
    if (argc != 9)
        return fail("usage");
    const bool bwd = std::strcmp(argv[1], "bwd") == 0;
    const int layout = std::atoi(argv[2]);
    const int dtype = std::atoi(argv[3]);
    const long long rows = std::atoll(argv[4]), cols = std::atoll(argv[5]);
    const long long ld_in = std::atoll(argv[6]), ld_out = std::atoll(argv[7]);
    const int mis = std::atoi(argv[8]);
    const int es = dtype == 0 ? 4 : 2;
    // fake, far-apart device addresses; nothing is dereferenced
    const uintptr_t A = (uintptr_t(1) << 44) + mis * es, B = uintptr_t(2) << 44, D = uintptr_t(3) << 44,
                    Y = uintptr_t(4) << 44, Z = uintptr_t(5) << 44;
    glu_status st;
    if (!bwd)
        st = glu_fwd(glu_kind(0), glu_layout(layout), glu_dtype(dtype), rows, cols, (void *)A, ld_in,
                     layout == 0 ? (void *)B : nullptr, ld_in, (void *)Y, ld_out, 0, nullptr);
    else
        st = glu_bwd(glu_kind(0), glu_layout(layout), glu_dtype(dtype), rows, cols, (void *)A, ld_in,
                     layout == 0 ? (void *)B : nullptr, ld_in, (const void *)D, ld_out, (void *)Y,
                     layout == 0 ? ld_out : ld_in, layout == 0 ? (void *)Z : nullptr, ld_out, 0, nullptr);
    if (st != GLU_OK)
        return fail("status", st);
    // expected operand bases / strides as the planner must use them
    const uintptr_t in0 = A, in1 = layout == 0 ? B : A + uintptr_t(cols) * es, out0 = Y;
    const long long ld_o = (bwd && layout == 1) ? ld_in : ld_out;   // gate_up dx has x's stride
    // Every launch covers rows [r0, r0+nrows) x columns [c0, c0+pcols) of the
    // problem (or a flat range when all strides equal cols and rows merge).
    const bool merged = layout == 0 && ld_in == cols && ld_out == cols;
    std::vector<std::pair<long long, long long>> iv;   // logical [begin, end) intervals
    for (size_t L = 0; L < glu::g_launches.size(); ++L) {
        const glu::Args &p = glu::g_launches[L];
        const int ve = glu::g_vec[L] ? (dtype == 0 ? 4 : 8) : 1;
        if (p.units == 0 || p.units >= (1u << 31))
            return fail("units range", p.units);
        if (p.cols == 0 || (long long)p.cols > (1ll << 31))
            return fail("cols range", p.cols);
        if ((long long)p.units_per_row * ve < (long long)p.cols ||
            (long long)(p.units_per_row - 1) * ve >= (long long)p.cols)
            return fail("units_per_row", p.units_per_row, p.cols);
        if (p.units % p.units_per_row != 0)
            return fail("units not whole rows", p.units, p.units_per_row);
        const long long nrows = p.units / p.units_per_row;
        const long long off0 = ((long long)((uintptr_t)p.in0 - in0)) / es;
        const long long off1 = ((long long)((uintptr_t)p.in1 - in1)) / es;
        const long long offo = ((long long)((uintptr_t)p.out0 - out0)) / es;
        // kernel index math at boundary units
        std::vector<uint32_t> us = {0u, p.units - 1, p.units_per_row - 1, p.units_per_row,
                                    p.units / 2, p.units - p.units_per_row};
        for (int k = 0; k < 31; ++k)
            if ((1u << k) < p.units) {
                us.push_back(1u << k);
                us.push_back((1u << k) - 1);
            }
        for (uint32_t u : us) {
            if (u >= p.units)
                continue;
            uint32_t r = (uint32_t)(((uint64_t)u * p.row_div.magic) >> 32);
            r = (r + u) >> p.row_div.shift;
            uint32_t col = (u - r * p.units_per_row) * uint32_t(ve);
            if ((long long)r >= nrows)
                return fail("row index", r, nrows);
            if ((long long)r != (long long)u / p.units_per_row)
                return fail("row division", u, r);
            if ((long long)col != ((long long)u % p.units_per_row) * ve)
                return fail("column index wrapped", u, col);
            if (col >= p.cols)
                return fail("column past row", col, p.cols);
        }
        if (merged) {
            if (nrows != 1 || off1 != off0 || offo != off0)
                return fail("merged launch offsets", off0, offo);
            iv.push_back({off0, off0 + (long long)p.cols});
        } else {
            const long long r0 = off0 / ld_in, c0 = off0 % ld_in;
            if (off1 != r0 * ld_in + c0 || offo != r0 * ld_o + c0)
                return fail("strided launch offsets", off1, offo);
            if (p.ld_in0 != ld_in || p.ld_out0 != ld_o)
                return fail("launch strides", p.ld_in0, p.ld_out0);
            if (r0 + nrows > rows || c0 + (long long)p.cols > cols)
                return fail("launch past the problem", r0 + nrows, c0 + p.cols);
            for (long long r = r0; r < r0 + nrows; ++r)
                iv.push_back({r * cols + c0, r * cols + c0 + (long long)p.cols});
        }
    }
    std::sort(iv.begin(), iv.end());
    long long at = 0;
    for (auto &x : iv) {
        if (x.first != at)
            return fail("gap or overlap at", at, x.first);
        at = x.second;
    }
    if (at != rows * cols)
        return fail("coverage", at, rows * cols);
    std::printf("ok %zu\n", glu::g_launches.size());
    return 0;
}
