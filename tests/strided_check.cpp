// Host-only check of the strided-operand planner in glu_api.cpp
// (glu_fwd_strided / glu_bwd_strided).
//
// Both launchers are replaced by stubs that record what would be enqueued.
// For one call the program reports which path was taken and checks it:
//   "rows"  -- streaming kernels on the row-major problem,
//   "cols"  -- streaming kernels on the transposed problem,
//   "tiles" -- the LDS-tiled kernel; the launches must cover every tile of
//              the (possibly transposed) problem exactly once, each launch
//              within the grid limit, with every operand's strides and the
//              access mode its strides and alignment allow; prints the
//              orientation and the modes (D direct, T transposed, G gather).
//
// usage: strided_check <fwd|bwd> <dtype> <rows> <cols> <rs cs> x (2 or 3 inputs + 1 or 2 outputs)
//                      [<in-place spec>]
// Operands sit at far-apart fake addresses (nothing is dereferenced) unless
// an in-place spec "o<k>=i<j>" places output k on input j.
// prints "<status> <path> <launches>" or "FAIL <reason>".
#include "glu.h"
#include "glu_internal.h"
#include "gemm_internal.h"
#include "rmsnorm_internal.h"

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

namespace glu {
static std::vector<Args> g_launches;
static std::vector<std::pair<TileArgs, uint32_t>> g_tiles;
hipError_t launch(int, int, bool, bool, const Args &args, hipStream_t)
{
    g_launches.push_back(args);
    return hipSuccess;
}
hipError_t launch_tiles(int, int, bool, const TileArgs &args, uint32_t ntiles, hipStream_t)
{
    g_tiles.push_back({args, ntiles});
    return hipSuccess;
}
hipError_t launch_gemm_glu(int, int, const GemmArgs &, hipStream_t)
{
    return hipSuccess;   // not exercised here
}
hipError_t launch_add_rmsnorm(int, bool, RmsShape, uint32_t, const RmsArgs &, hipStream_t)
{
    return hipSuccess;
}
}  // namespace glu

static int fail(const char *why, long long a = 0, long long b = 0)
{
    std::printf("FAIL %s %lld %lld\n", why, a, b);
    return 1;
}

int main(int argc, char **argv)
{
    if (argc < 5)
        return fail("usage");
    const bool bwd = std::strcmp(argv[1], "bwd") == 0;
    const int dtype = std::atoi(argv[2]);
    const long long rows = std::atoll(argv[3]), cols = std::atoll(argv[4]);
    const int nin = bwd ? 3 : 2, nout = bwd ? 2 : 1, nops = nin + nout;
    if (argc < 5 + 2 * nops)
        return fail("usage");
    long long rs[5], cs[5];
    uintptr_t p[5];
    for (int i = 0; i < nops; ++i) {
        rs[i] = std::atoll(argv[5 + 2 * i]);
        cs[i] = std::atoll(argv[6 + 2 * i]);
        p[i] = uintptr_t(i + 1) << 52;
    }
    for (int k = 5 + 2 * nops; k < argc; ++k) {
        int o, j;
        if (std::sscanf(argv[k], "o%d=i%d", &o, &j) == 2)
            p[nin + o] = p[j];
        else if (std::sscanf(argv[k], "i%d+%d", &j, &o) == 2)   // input j offset by o elements from input 0
            p[j] = p[0] + uintptr_t(o) * (dtype == 0 ? 4 : 2);
        else if (std::sscanf(argv[k], "o%d+%d", &j, &o) == 2)   // output j offset by o elements from input 0
            p[nin + j] = p[0] + uintptr_t(o) * (dtype == 0 ? 4 : 2);
    }
    glu_status st;
    if (!bwd)
        st = glu_fwd_strided(glu_kind(0), glu_dtype(dtype), rows, cols, (void *)p[0], rs[0], cs[0], (void *)p[1],
                             rs[1], cs[1], (void *)p[2], rs[2], cs[2], nullptr);
    else
        st = glu_bwd_strided(glu_kind(0), glu_dtype(dtype), rows, cols, (void *)p[0], rs[0], cs[0], (void *)p[1],
                             rs[1], cs[1], (void *)p[2], rs[2], cs[2], (void *)p[3], rs[3], cs[3], (void *)p[4],
                             rs[4], cs[4], nullptr);
    if (st != GLU_OK) {
        std::printf("%d none 0\n", int(st));
        return 0;
    }
    if (!glu::g_launches.empty() && !glu::g_tiles.empty())
        return fail("mixed paths");
    if (glu::g_launches.empty() && glu::g_tiles.empty()) {
        if (rows * cols != 0)
            return fail("nothing launched");
        std::printf("0 none 0\n");
        return 0;
    }
    if (!glu::g_tiles.empty()) {
        // the kernel computes in row orientation: the problem is transposed
        // when more operands are column-contiguous than row-contiguous
        int nrow = 0, ncol = 0;
        for (int i = 0; i < nops; ++i) {
            nrow += cs[i] == 1;
            ncol += rs[i] == 1;
        }
        const bool flip = ncol > nrow;
        const long long R = flip ? cols : rows, C = flip ? rows : cols;
        const long long tr = (R + glu::kTile - 1) / glu::kTile, tc = (C + glu::kTile - 1) / glu::kTile;
        const int es = dtype == 0 ? 4 : 2;
        long long next = 0;
        std::string modes;
        for (auto &L : glu::g_tiles) {
            const glu::TileArgs &t = L.first;
            if (L.second == 0 || L.second > glu::kMaxTilesPerLaunch)
                return fail("tiles per launch", L.second);
            if ((long long)t.tile0 != next)
                return fail("tile order", t.tile0, next);
            next += L.second;
            if (t.rows != R || t.cols != C || (long long)t.tiles_r != tr || (long long)t.tiles_c != tc)
                return fail("tile shape", t.rows, t.tiles_c);
            modes.clear();
            for (int i = 0; i < nops; ++i) {
                const bool in = i < nin;
                const uintptr_t ptr = in ? (uintptr_t)t.in[i] : (uintptr_t)t.out[i - nin];
                const long long grs = in ? t.irs[i] : t.ors[i - nin], gcs = in ? t.ics[i] : t.ocs[i - nin];
                const int m = in ? t.in_mode[i] : t.out_mode[i - nin];
                const long long wrs = flip ? cs[i] : rs[i], wcs = flip ? rs[i] : cs[i];
                if (ptr != p[i] || grs != wrs || gcs != wcs)
                    return fail("operand", i);
                // 16-byte chunks: along the row (direct) need a column stride
                // of 1 and every chunk start 16-byte aligned; down the column
                // (transposed) the same with the roles swapped
                const bool base16 = (ptr & 15) == 0;
                const bool can_d = wcs == 1 && base16 && (R <= 1 || (wrs * es) % 16 == 0);
                const bool can_t = wrs == 1 && base16 && (C <= 1 || (wcs * es) % 16 == 0);
                const int want = can_d ? glu::kDirect : can_t ? glu::kTransposed : glu::kGather;
                if (m != want)
                    return fail("mode", i, m);
                modes += "DTG"[m];
            }
        }
        if (next != tr * tc)
            return fail("tile coverage", next, tr * tc);
        {
            // LDS slots: distinct per transposed input, distinct per
            // transposed output, all below nslots, nslots no larger than needed
            const glu::TileArgs &t = glu::g_tiles[0].first;
            int nti = 0, nto = 0, used_i = 0, used_o = 0;
            for (int i = 0; i < nin; ++i)
                if (t.in_mode[i] == glu::kTransposed) {
                    ++nti;
                    if (t.in_slot[i] >= t.nslots || (used_i >> t.in_slot[i]) & 1)
                        return fail("input slot", i, t.in_slot[i]);
                    used_i |= 1 << t.in_slot[i];
                }
            for (int i = 0; i < nout; ++i)
                if (t.out_mode[i] == glu::kTransposed) {
                    ++nto;
                    if (t.out_slot[i] >= t.nslots || (used_o >> t.out_slot[i]) & 1)
                        return fail("output slot", i, t.out_slot[i]);
                    used_o |= 1 << t.out_slot[i];
                }
            if (t.nslots != (nti > nto ? nti : nto))
                return fail("slot count", t.nslots);
        }
        if (tr * tc <= (1ll << 24)) {
            // the launch order visits every tile exactly once
            std::vector<unsigned char> seen(size_t(tr * tc), 0);
            for (long long i = 0; i < tr * tc; ++i) {
                const glu::TileCoord c = glu::tile_coord(uint32_t(i), uint32_t(tr), uint32_t(tc));
                if ((long long)c.r >= tr || (long long)c.c >= tc)
                    return fail("tile outside the grid", c.r, c.c);
                if (seen[size_t(c.r * tc + c.c)]++)
                    return fail("tile visited twice", c.r, c.c);
            }
        }
        std::printf("0 tiles %zu %s %s\n", glu::g_tiles.size(), flip ? "flip" : "keep", modes.c_str());
        return 0;
    }
    // streaming path: which orientation, and every operand's leading stride
    const glu::Args &a = glu::g_launches.at(0);
    const bool transposed = (uintptr_t)a.in0 == p[0] && cols > 1 && rows > 1 && cs[0] != 1;
    const long long *lead = transposed ? cs : rs;
    const long long R = transposed ? cols : rows, C = transposed ? rows : cols;
    const long long lds[5] = {a.ld_in0, a.ld_in1, a.ld_in2, a.ld_out0, a.ld_out1};
    const int idx[5] = {0, 1, 2, 3, 4};
    for (int i = 0; i < nops; ++i) {
        const int k = i < nin ? idx[i] : 3 + (i - nin);
        const long long want = R > 1 ? lead[i] : C;
        if (lds[k] != want)
            return fail("leading stride", i, lds[k]);
    }
    long long covered = 0;
    for (auto &L : glu::g_launches)
        covered += (long long)(L.units / L.units_per_row) * L.cols;
    if (covered != R * C)
        return fail("coverage", covered, R * C);
    std::printf("0 %s %zu\n", transposed ? "cols" : "rows", glu::g_launches.size());
    return 0;
}
