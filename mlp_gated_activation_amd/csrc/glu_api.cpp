// glu_api.cpp -- host side of the C ABI declared in include/glu.h:
// argument validation (entirely before any HIP call), aliasing analysis,
// and launch planning.
//
// Sources (page title -- section):
//   [SWIGLU] "Write a Triton SiLU-Mul (SwiGLU) Kernel"
//   [LIGER]  "Kernel Profile: SwiGLU (Tier 1 -- Element-wise)"
#include "glu.h"

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "glu_internal.h"
#include "gemm_internal.h"
#include "rmsnorm_internal.h"

namespace {

using glu::Args;

// A strided operand: `rows` rows of `width` elements, `ld` elements apart,
// starting at byte address `p`.
struct Region {
    uintptr_t p;
    int64_t ld;
    int64_t width;
};

// Byte extent [p, p + extent) of a region; false on int64 overflow.
bool extent_bytes(int64_t rows, const Region &r, int esize, int64_t *out)
{
    int64_t span;
    if (__builtin_mul_overflow(rows - 1, r.ld, &span))
        return false;
    if (__builtin_add_overflow(span, r.width, &span))
        return false;
    if (__builtin_mul_overflow(span, int64_t(esize), &span))
        return false;
    uintptr_t end;
    if (__builtin_add_overflow(r.p, uintptr_t(span), &end))
        return false;
    *out = span;
    return true;
}

int64_t floor_div(int64_t a, int64_t b)  // b > 0
{
    int64_t q = a / b;
    return (a % b != 0 && a < 0) ? q - 1 : q;
}

// True when some element of region x and some element of region y share a
// byte.  Exact for equal strides; conservative (true) when the byte extents
// intersect and the strides differ.
bool overlaps(int64_t rows, const Region &x, const Region &y, int esize)
{
    int64_t ex = 0, ey = 0;
    extent_bytes(rows, x, esize, &ex);
    extent_bytes(rows, y, esize, &ey);
    if (x.p + uintptr_t(ex) <= y.p || y.p + uintptr_t(ey) <= x.p)
        return false;
    if (x.ld != y.ld)
        return true;
    // Rows i of x and i + k of y overlap iff -wy < d + k*L < wx  (bytes),
    // d = y.p - x.p, L = ld * esize.
    const int64_t L = x.ld * esize;
    const int64_t d = int64_t(y.p - x.p);
    const int64_t wx = x.width * esize, wy = y.width * esize;
    int64_t klo = floor_div(-wy - d, L) + 1;         // smallest k with d + kL > -wy
    int64_t khi = -floor_div(-(wx - d), L) - 1;      // largest k with d + kL < wx
    if (klo < -(rows - 1))
        klo = -(rows - 1);
    if (khi > rows - 1)
        khi = rows - 1;
    return klo <= khi;
}

bool same(const Region &x, const Region &y) { return x.p == y.p && x.ld == y.ld && x.width == y.width; }

// An output may coincide exactly with an input, never partially.
bool bad_alias(int64_t rows, const Region &out, const Region *ins, int nin, int esize)
{
    for (int i = 0; i < nin; ++i)
        if (!same(out, ins[i]) && overlaps(rows, out, ins[i], esize))
            return true;
    return false;
}

bool aligned16(uintptr_t p) { return (p & 15u) == 0; }

// Enqueue launches covering `rows` x `cols` elements.  When every operand is
// a dense (ld == cols) matrix the rows are merged into one long row.
glu_status enqueue(int dtype, int kind, bool bwd, int64_t rows, int64_t cols, Args a, bool vec,
                   hipStream_t stream)
{
    const int es = glu::elem_size(dtype);
    const int ve = vec ? glu::vec_elems(dtype) : 1;
    const int nin = bwd ? 3 : 2;
    const int nout = bwd ? 2 : 1;
    const int64_t *lds[5] = {&a.ld_in0, &a.ld_in1, &a.ld_in2, &a.ld_out0, &a.ld_out1};
    const bool used[5] = {true, true, nin == 3, true, nout == 2};
    bool dense = true;
    for (int i = 0; i < 5; ++i)
        if (used[i] && *lds[i] != cols)
            dense = false;
    if (dense && rows > 1) {
        cols *= rows;
        rows = 1;
    }
    const int64_t upr = (cols + ve - 1) / ve;   // units per row
    const void *ins[3] = {a.in0, a.in1, a.in2};
    void *outs[2] = {a.out0, a.out1};

    auto run = [&](int64_t r0, int64_t nrows, int64_t c0, int64_t ncols) -> glu_status {
        Args p = a;
        const int64_t u = (ncols + ve - 1) / ve;
        for (int i = 0; i < nin; ++i)
            (&p.in0)[i] = static_cast<const char *>(ins[i]) + (r0 * *lds[i] + c0) * es;
        for (int i = 0; i < nout; ++i)
            (&p.out0)[i] = static_cast<char *>(outs[i]) + (r0 * *lds[3 + i] + c0) * es;
        p.units = uint32_t(nrows * u);
        p.units_per_row = uint32_t(u);
        p.cols = uint32_t(ncols);
        p.row_div = glu::make_divider(uint32_t(u));
        return glu::launch(dtype, kind, bwd, vec, p, stream) == hipSuccess ? GLU_OK : GLU_ERR_HIP;
    };

    // Each launch covers at most kMaxUnitsPerLaunch units and rows of at most
    // max_cols elements (32-bit column indices in the kernel).
    const int64_t maxu = glu::kMaxUnitsPerLaunch;
    const int64_t max_cols = glu::kMaxColsPerLaunch < maxu * ve ? glu::kMaxColsPerLaunch : maxu * ve;
    if (cols <= max_cols) {
        const int64_t rows_per = maxu / upr;   // >= 1 since upr <= max_cols / ve <= maxu
        for (int64_t r0 = 0; r0 < rows; r0 += rows_per) {
            int64_t n = rows - r0 < rows_per ? rows - r0 : rows_per;
            glu_status s = run(r0, n, 0, cols);
            if (s != GLU_OK)
                return s;
        }
    } else {
        // rows longer than one launch: split each into column chunks
        for (int64_t r0 = 0; r0 < rows; ++r0)
            for (int64_t c0 = 0; c0 < cols; c0 += max_cols) {
                glu_status s = run(r0, 1, c0, cols - c0 < max_cols ? cols - c0 : max_cols);
                if (s != GLU_OK)
                    return s;
            }
    }
    return GLU_OK;
}

bool valid_enums(int kind, int layout, int dtype)
{
    return kind >= GLU_SILU && kind <= GLU_RELU && layout >= GLU_SEPARATE && layout <= GLU_GATE_UP &&
           dtype >= GLU_F32 && dtype <= GLU_BF16;
}

// Shared checks of the input side; fills the a and b regions.
glu_status check_inputs(glu_layout layout, int es, int64_t rows, int64_t cols, void *a, int64_t lda,
                        void *b, int64_t ldb, Region *ra, Region *rb)
{
    if (a == nullptr)
        return GLU_ERR_NULL;
    if (layout == GLU_SEPARATE) {
        if (b == nullptr)
            return GLU_ERR_NULL;
        if (lda < cols || ldb < cols)
            return GLU_ERR_STRIDE;
        *ra = Region{uintptr_t(a), lda, cols};
        *rb = Region{uintptr_t(b), ldb, cols};
    } else {
        if (b != nullptr)
            return GLU_ERR_NULL;
        int64_t two;
        if (__builtin_mul_overflow(cols, int64_t(2), &two))
            return GLU_ERR_SHAPE;
        if (lda < two)
            return GLU_ERR_STRIDE;
        *ra = Region{uintptr_t(a), lda, cols};
        *rb = Region{uintptr_t(a) + uintptr_t(cols) * es, lda, cols};
        int64_t ext;
        if (!extent_bytes(rows, Region{uintptr_t(a), lda, two}, es, &ext))
            return GLU_ERR_SHAPE;
    }
    int64_t ext;
    if (!extent_bytes(rows, *ra, es, &ext) || !extent_bytes(rows, *rb, es, &ext))
        return GLU_ERR_SHAPE;
    return GLU_OK;
}

bool vec_ok(const Region *r, int n, int es, int64_t rows)
{
    for (int i = 0; i < n; ++i) {
        if (!aligned16(r[i].p))
            return false;
        if (rows > 1 && ((r[i].ld * es) & 15) != 0)
            return false;
    }
    return true;
}

// --- strided operands -------------------------------------------------------

struct Op2 {
    uintptr_t p;
    int64_t rs, cs;
};

bool same2(const Op2 &x, const Op2 &y) { return x.p == y.p && x.rs == y.rs && x.cs == y.cs; }

// Byte extent of an operand's elements: [p, p + span); false on overflow.
bool span2(int64_t rows, int64_t cols, const Op2 &o, int es, int64_t *out)
{
    int64_t a, b, s;
    if (__builtin_mul_overflow(rows - 1, o.rs, &a) || __builtin_mul_overflow(cols - 1, o.cs, &b) ||
        __builtin_add_overflow(a, b, &s) || __builtin_add_overflow(s, int64_t(1), &s) ||
        __builtin_mul_overflow(s, int64_t(es), &s))
        return false;
    uintptr_t end;
    if (__builtin_add_overflow(o.p, uintptr_t(s), &end))
        return false;
    *out = s;
    return true;
}

// (r, c) -> r*rs + c*cs is one-to-one on [0, rows) x [0, cols) (sufficient
// condition: the larger stride steps over the whole extent of the smaller).
bool injective(int64_t rows, int64_t cols, const Op2 &o)
{
    int64_t s1 = o.rs, n1 = rows, s2 = o.cs, n2 = cols;
    if (n1 == 1)
        return n2 == 1 || s2 >= 1;
    if (n2 == 1)
        return s1 >= 1;
    if (s1 > s2) {
        int64_t t = s1; s1 = s2; s2 = t;
        t = n1; n1 = n2; n2 = t;
    }
    int64_t need;
    return s1 >= 1 && !__builtin_mul_overflow(s1, n1, &need) && s2 >= need;
}

// The operand as `n` runs of `width` contiguous elements `ld` apart: row-major
// (column stride 1) gives rows of cols, column-major (row stride 1) gives
// columns of rows.  Returns 0 when it is neither, 1 row-major, 2 column-major.
int as_runs(int64_t rows, int64_t cols, const Op2 &o, int64_t *n, Region *r)
{
    if ((cols == 1 || o.cs == 1) && (rows == 1 || o.rs >= cols)) {
        *n = rows;
        *r = Region{o.p, rows > 1 ? o.rs : cols, cols};
        return 1;
    }
    if ((rows == 1 || o.rs == 1) && (cols == 1 || o.cs >= rows)) {
        *n = cols;
        *r = Region{o.p, cols > 1 ? o.cs : rows, rows};
        return 2;
    }
    return 0;
}

// True when some element of x and some element of y share a byte.  Exact
// for two views with the same orientation and leading stride (for example
// the two halves of [gate | up]); conservative (true) otherwise when the
// byte extents intersect.
bool overlap2(int64_t rows, int64_t cols, const Op2 &x, const Op2 &y, int es)
{
    int64_t ex = 0, ey = 0;
    span2(rows, cols, x, es, &ex);
    span2(rows, cols, y, es, &ey);
    if (x.p + uintptr_t(ex) <= y.p || y.p + uintptr_t(ey) <= x.p)
        return false;
    int64_t nx, ny;
    Region rx, ry;
    const int ox = as_runs(rows, cols, x, &nx, &rx), oy = as_runs(rows, cols, y, &ny, &ry);
    if (ox == 0 || ox != oy)
        return true;
    return overlaps(nx, rx, ry, es);
}

glu_status strided(bool bwd, int kind, int dtype, int64_t rows, int64_t cols, const Op2 *ins, const Op2 *outs,
                   hipStream_t stream)
{
    if (!(kind >= GLU_SILU && kind <= GLU_RELU) || !(dtype >= GLU_F32 && dtype <= GLU_BF16))
        return GLU_ERR_ENUM;
    if (rows < 0 || cols < 0)
        return GLU_ERR_SHAPE;
    if (rows == 0 || cols == 0)
        return GLU_OK;
    const int nin = bwd ? 3 : 2, nout = bwd ? 2 : 1;
    const int es = glu::elem_size(dtype);
    for (int i = 0; i < nin + nout; ++i) {
        const Op2 &o = i < nin ? ins[i] : outs[i - nin];
        if (o.p == 0)
            return GLU_ERR_NULL;
        if (o.rs < 0 || o.cs < 0)
            return GLU_ERR_STRIDE;
        if (o.p % uintptr_t(es) != 0)
            return GLU_ERR_ARG;
        int64_t ext;
        if (!span2(rows, cols, o, es, &ext))
            return GLU_ERR_SHAPE;
    }
    for (int k = 0; k < nout; ++k) {
        if (!injective(rows, cols, outs[k]))
            return GLU_ERR_STRIDE;
        for (int i = 0; i < nin; ++i)
            if (!same2(outs[k], ins[i]) && overlap2(rows, cols, outs[k], ins[i], es))
                return GLU_ERR_ALIAS;
    }
    if (nout == 2 && overlap2(rows, cols, outs[0], outs[1], es))
        return GLU_ERR_ALIAS;

    // Row-major everywhere (column stride 1, rows apart): the streaming kernels.
    // Column-major everywhere: the same kernels on the transposed problem.
    for (int transpose = 0; transpose < 2; ++transpose) {
        const int64_t R = transpose ? cols : rows, C = transpose ? rows : cols;
        bool ok = true;
        Region rin[3], rout[2];
        for (int i = 0; i < nin + nout; ++i) {
            const Op2 &o = i < nin ? ins[i] : outs[i - nin];
            const int64_t unit = transpose ? o.rs : o.cs, ld = transpose ? o.cs : o.rs;
            if ((C > 1 && unit != 1) || (R > 1 && ld < C))
                ok = false;
            const Region r{o.p, R > 1 ? ld : C, C};
            (i < nin ? rin[i] : rout[i - nin]) = r;
        }
        if (!ok)
            continue;
        Region all[5];
        for (int i = 0; i < nin; ++i)
            all[i] = rin[i];
        for (int i = 0; i < nout; ++i)
            all[nin + i] = rout[i];
        Args p{};
        p.in0 = reinterpret_cast<const void *>(rin[0].p);
        p.in1 = reinterpret_cast<const void *>(rin[1].p);
        p.in2 = bwd ? reinterpret_cast<const void *>(rin[2].p) : nullptr;
        p.out0 = reinterpret_cast<void *>(rout[0].p);
        p.out1 = bwd ? reinterpret_cast<void *>(rout[1].p) : nullptr;
        p.ld_in0 = rin[0].ld;
        p.ld_in1 = rin[1].ld;
        p.ld_in2 = bwd ? rin[2].ld : 0;
        p.ld_out0 = rout[0].ld;
        p.ld_out1 = bwd ? rout[1].ld : 0;
        return enqueue(dtype, kind, bwd, R, C, p, vec_ok(all, nin + nout, es, R), stream);
    }

    // Mixed layouts: 64 x 64 tiles.  The kernel works in row orientation, so
    // the whole problem is transposed when more operands are contiguous down
    // the columns than along the rows.
    int nrow = 0, ncol = 0;
    for (int i = 0; i < nin + nout; ++i) {
        const Op2 &o = i < nin ? ins[i] : outs[i - nin];
        nrow += o.cs == 1;
        ncol += o.rs == 1;
    }
    const bool flip = ncol > nrow;
    const int64_t R = flip ? cols : rows, C = flip ? rows : cols;
    const int64_t tr = (R + glu::kTile - 1) / glu::kTile, tc = (C + glu::kTile - 1) / glu::kTile;
    int64_t ntiles;
    if (__builtin_mul_overflow(tr, tc, &ntiles) || ntiles > int64_t(UINT32_MAX))
        return GLU_ERR_SHAPE;
    auto mode = [&](const Op2 &o, int64_t *rs, int64_t *cs) -> uint8_t {
        *rs = flip ? o.cs : o.rs;
        *cs = flip ? o.rs : o.cs;
        const bool base16 = aligned16(o.p);
        if (*cs == 1 && base16 && (R <= 1 || ((*rs * es) & 15) == 0))
            return glu::kDirect;
        if (*rs == 1 && base16 && (C <= 1 || ((*cs * es) & 15) == 0))
            return glu::kTransposed;
        return glu::kGather;
    };
    glu::TileArgs t{};
    for (int i = 0; i < nin; ++i) {
        t.in[i] = reinterpret_cast<const void *>(ins[i].p);
        t.in_mode[i] = mode(ins[i], &t.irs[i], &t.ics[i]);
    }
    for (int i = 0; i < nout; ++i) {
        t.out[i] = reinterpret_cast<void *>(outs[i].p);
        t.out_mode[i] = mode(outs[i], &t.ors[i], &t.ocs[i]);
    }
    // LDS slots: transposed inputs first; outputs reuse them after the math
    int nti = 0, nto = 0;
    for (int i = 0; i < nin; ++i)
        if (t.in_mode[i] == glu::kTransposed)
            t.in_slot[i] = uint8_t(nti++);
    for (int i = 0; i < nout; ++i)
        if (t.out_mode[i] == glu::kTransposed)
            t.out_slot[i] = uint8_t(nto++);
    t.nslots = uint8_t(nti > nto ? nti : nto);
    t.rows = R;
    t.cols = C;
    t.tiles_r = uint32_t(tr);
    t.tiles_c = uint32_t(tc);
    for (int64_t t0 = 0; t0 < ntiles; t0 += glu::kMaxTilesPerLaunch) {
        const int64_t n = ntiles - t0 < glu::kMaxTilesPerLaunch ? ntiles - t0 : glu::kMaxTilesPerLaunch;
        t.tile0 = uint32_t(t0);
        if (glu::launch_tiles(dtype, kind, bwd, t, uint32_t(n), stream) != hipSuccess)
            return GLU_ERR_HIP;
    }
    return GLU_OK;
}

}  // namespace

extern "C" {

glu_status glu_gemm_fwd(glu_kind kind, glu_dtype dtype, int64_t M, int64_t N, int64_t K, const void *x,
                        int64_t ldx, const void *w_gate, int64_t ldwg, const void *w_up, int64_t ldwu, void *h,
                        int64_t ldh, void *gu, int64_t ldgu, hipStream_t stream)
{
    if (!(kind >= GLU_SILU && kind <= GLU_RELU) || !(dtype == GLU_F16 || dtype == GLU_BF16))
        return GLU_ERR_ENUM;
    if (M < 0 || N < 0 || K < 0 || M > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
        return GLU_ERR_SHAPE;
    if (M == 0 || N == 0)
        return GLU_OK;
    if (h == nullptr)
        return GLU_ERR_NULL;
    if (K == 0) {
        // h = act(0) * 0: the inputs are never read
        x = w_gate = w_up = nullptr;
        ldx = ldwg = ldwu = 0;
    } else if (x == nullptr || w_gate == nullptr || w_up == nullptr) {
        return GLU_ERR_NULL;
    }
    int64_t two_n = 2 * N;
    if (ldx < K || ldwg < K || ldwu < K || ldh < N || (gu != nullptr && ldgu < two_n))
        return GLU_ERR_STRIDE;
    const int es = 2;
    const uintptr_t px = uintptr_t(x), pg = uintptr_t(w_gate), pu = uintptr_t(w_up), ph = uintptr_t(h),
                    pgu = uintptr_t(gu);
    if (!aligned16(px) || !aligned16(pg) || !aligned16(pu) || (K & 7) || (ldx & 7) || (ldwg & 7) || (ldwu & 7) ||
        (ph & 1) || (pgu & 1))
        return GLU_ERR_ARG;
    const int64_t in_rows = K == 0 ? 0 : 1;   // inputs take no bytes when K == 0
    const int cfg = glu::gemm_config(M);
    const int64_t bm = glu::kGemmTiles[cfg].bm, bn = glu::kGemmTiles[cfg].bn;
    const int64_t tm = (M + bm - 1) / bm, tn = (N + bn - 1) / bn;
    if (tm * tn > int64_t(glu::kMaxGemmTiles) || ldx >= glu::kGemmMaxLd || ldwg >= glu::kGemmMaxLd ||
        ldwu >= glu::kGemmMaxLd)
        return GLU_ERR_SHAPE;
    // byte extents of every operand (overflow -> shape error)
    const Region rx{px, ldx, K}, rg{pg, ldwg, K}, ru{pu, ldwu, K}, rh{ph, ldh, N}, rgu{pgu, ldgu, two_n};
    int64_t ex, eg, eu, eh, egu = 0;
    if (!extent_bytes(M, rx, es, &ex) || !extent_bytes(N, rg, es, &eg) || !extent_bytes(N, ru, es, &eu) ||
        !extent_bytes(M, rh, es, &eh) || (gu != nullptr && !extent_bytes(M, rgu, es, &egu)))
        return GLU_ERR_SHAPE;
    ex *= in_rows;
    eg *= in_rows;
    eu *= in_rows;
    auto apart = [](uintptr_t a, int64_t ea, uintptr_t b, int64_t eb) {
        return a + uintptr_t(ea) <= b || b + uintptr_t(eb) <= a;
    };
    if (!apart(ph, eh, px, ex) || !apart(ph, eh, pg, eg) || !apart(ph, eh, pu, eu))
        return GLU_ERR_ALIAS;
    if (gu != nullptr && (!apart(pgu, egu, px, ex) || !apart(pgu, egu, pg, eg) || !apart(pgu, egu, pu, eu) ||
                          overlaps(M, rh, Region{pgu, ldgu, two_n}, es)))
        return GLU_ERR_ALIAS;
    glu::GemmArgs a{};
    a.x = x;
    a.wg = w_gate;
    a.wu = w_up;
    a.h = h;
    a.gu = gu;
    a.ldx = ldx;
    a.ldwg = ldwg;
    a.ldwu = ldwu;
    a.ldh = ldh;
    a.ldgu = ldgu;
    a.M = int32_t(M);
    a.N = int32_t(N);
    a.K = int32_t(K);
    a.tiles_m = uint32_t(tm);
    a.tiles_n = uint32_t(tn);
    a.config = cfg;
    return glu::launch_gemm_glu(dtype, kind, a, stream) == hipSuccess ? GLU_OK : GLU_ERR_HIP;
}

glu_status glu_fwd_strided(glu_kind kind, glu_dtype dtype, int64_t rows, int64_t cols, const void *a, int64_t a_rs,
                           int64_t a_cs, const void *b, int64_t b_rs, int64_t b_cs, void *y, int64_t y_rs,
                           int64_t y_cs, hipStream_t stream)
{
    const Op2 ins[2] = {{uintptr_t(a), a_rs, a_cs}, {uintptr_t(b), b_rs, b_cs}};
    const Op2 outs[1] = {{uintptr_t(y), y_rs, y_cs}};
    return strided(false, kind, dtype, rows, cols, ins, outs, stream);
}

glu_status glu_bwd_strided(glu_kind kind, glu_dtype dtype, int64_t rows, int64_t cols, const void *a, int64_t a_rs,
                           int64_t a_cs, const void *b, int64_t b_rs, int64_t b_cs, const void *dy,
                           int64_t dy_rs, int64_t dy_cs, void *da, int64_t da_rs, int64_t da_cs, void *db,
                           int64_t db_rs, int64_t db_cs, hipStream_t stream)
{
    const Op2 ins[3] = {{uintptr_t(a), a_rs, a_cs}, {uintptr_t(b), b_rs, b_cs}, {uintptr_t(dy), dy_rs, dy_cs}};
    const Op2 outs[2] = {{uintptr_t(da), da_rs, da_cs}, {uintptr_t(db), db_rs, db_cs}};
    return strided(true, kind, dtype, rows, cols, ins, outs, stream);
}


glu_status glu_fwd(glu_kind kind, glu_layout layout, glu_dtype dtype, int64_t rows, int64_t cols, void *a,
                   int64_t lda, void *b, int64_t ldb, void *y, int64_t ldy, int inplace, hipStream_t stream)
{
    if (!valid_enums(kind, layout, dtype))
        return GLU_ERR_ENUM;
    if (inplace != 0 && inplace != 1)
        return GLU_ERR_INPLACE;
    if (rows < 0 || cols < 0)
        return GLU_ERR_SHAPE;
    if (rows == 0 || cols == 0)
        return GLU_OK;
    if (rows > INT32_MAX)
        return GLU_ERR_SHAPE;
    const int es = glu::elem_size(dtype);
    Region ra, rb;
    glu_status s = check_inputs(layout, es, rows, cols, a, lda, b, ldb, &ra, &rb);
    if (s != GLU_OK)
        return s;
    Region ry;
    if (inplace) {
        if (y != nullptr)
            return GLU_ERR_INPLACE;
        ry = rb;   // [SWIGLU] Inputs, item 7: y may overwrite b
        // a may coincide with b exactly, but a partial overlap would let one
        // lane's store land on an element another lane still reads as a
        const Region ins[1] = {ra};
        if (bad_alias(rows, ry, ins, 1, es))
            return GLU_ERR_ALIAS;
    } else {
        if (y == nullptr)
            return GLU_ERR_NULL;
        if (ldy < cols)
            return GLU_ERR_STRIDE;
        ry = Region{uintptr_t(y), ldy, cols};
        int64_t ext;
        if (!extent_bytes(rows, ry, es, &ext))
            return GLU_ERR_SHAPE;
        const Region ins[2] = {ra, rb};
        if (bad_alias(rows, ry, ins, 2, es))
            return GLU_ERR_ALIAS;
    }
    const Region all[3] = {ra, rb, ry};
    const bool vec = vec_ok(all, 3, es, rows);
    Args p{};
    p.in0 = reinterpret_cast<const void *>(ra.p);
    p.in1 = reinterpret_cast<const void *>(rb.p);
    p.in2 = nullptr;
    p.out0 = reinterpret_cast<void *>(ry.p);
    p.out1 = nullptr;
    p.ld_in0 = ra.ld;
    p.ld_in1 = rb.ld;
    p.ld_in2 = 0;
    p.ld_out0 = ry.ld;
    p.ld_out1 = 0;
    return enqueue(dtype, kind, false, rows, cols, p, vec, stream);
}

glu_status glu_bwd(glu_kind kind, glu_layout layout, glu_dtype dtype, int64_t rows, int64_t cols, void *a,
                   int64_t lda, void *b, int64_t ldb, const void *dy, int64_t lddy, void *da, int64_t ldda,
                   void *db, int64_t lddb, int inplace, hipStream_t stream)
{
    if (!valid_enums(kind, layout, dtype))
        return GLU_ERR_ENUM;
    if (inplace != 0 && inplace != 1)
        return GLU_ERR_INPLACE;
    if (rows < 0 || cols < 0)
        return GLU_ERR_SHAPE;
    if (rows == 0 || cols == 0)
        return GLU_OK;
    if (rows > INT32_MAX)
        return GLU_ERR_SHAPE;
    const int es = glu::elem_size(dtype);
    Region ra, rb;
    glu_status s = check_inputs(layout, es, rows, cols, a, lda, b, ldb, &ra, &rb);
    if (s != GLU_OK)
        return s;
    if (dy == nullptr)
        return GLU_ERR_NULL;
    if (lddy < cols)
        return GLU_ERR_STRIDE;
    const Region rdy{uintptr_t(dy), lddy, cols};
    int64_t ext;
    if (!extent_bytes(rows, rdy, es, &ext))
        return GLU_ERR_SHAPE;
    Region rda, rdb;
    if (inplace) {
        // [LIGER] Key Patterns: gradients written over the saved a and b
        if (da != nullptr || db != nullptr)
            return GLU_ERR_INPLACE;
        rda = ra;
        rdb = rb;
        // dy must not overlap the outputs unless it is exactly one of them
        const Region outs[2] = {rda, rdb};
        for (int i = 0; i < 2; ++i)
            if (!same(outs[i], rdy) && overlaps(rows, outs[i], rdy, es))
                return GLU_ERR_ALIAS;
    } else {
        if (da == nullptr)
            return GLU_ERR_NULL;
        if (layout == GLU_SEPARATE) {
            if (db == nullptr)
                return GLU_ERR_NULL;
            if (ldda < cols || lddb < cols)
                return GLU_ERR_STRIDE;
            rda = Region{uintptr_t(da), ldda, cols};
            rdb = Region{uintptr_t(db), lddb, cols};
        } else {
            if (db != nullptr)
                return GLU_ERR_NULL;
            if (ldda < 2 * cols)
                return GLU_ERR_STRIDE;
            rda = Region{uintptr_t(da), ldda, cols};
            rdb = Region{uintptr_t(da) + uintptr_t(cols) * es, ldda, cols};
            if (!extent_bytes(rows, Region{uintptr_t(da), ldda, 2 * cols}, es, &ext))
                return GLU_ERR_SHAPE;
        }
        if (!extent_bytes(rows, rda, es, &ext) || !extent_bytes(rows, rdb, es, &ext))
            return GLU_ERR_SHAPE;
        const Region ins[3] = {ra, rb, rdy};
        if (bad_alias(rows, rda, ins, 3, es) || bad_alias(rows, rdb, ins, 3, es))
            return GLU_ERR_ALIAS;
    }
    if (overlaps(rows, rda, rdb, es))
        return GLU_ERR_ALIAS;
    const Region all[5] = {ra, rb, rdy, rda, rdb};
    const bool vec = vec_ok(all, 5, es, rows);
    Args p{};
    p.in0 = reinterpret_cast<const void *>(ra.p);
    p.in1 = reinterpret_cast<const void *>(rb.p);
    p.in2 = reinterpret_cast<const void *>(rdy.p);
    p.out0 = reinterpret_cast<void *>(rda.p);
    p.out1 = reinterpret_cast<void *>(rdb.p);
    p.ld_in0 = ra.ld;
    p.ld_in1 = rb.ld;
    p.ld_in2 = rdy.ld;
    p.ld_out0 = rda.ld;
    p.ld_out1 = rdb.ld;
    return enqueue(dtype, kind, true, rows, cols, p, vec, stream);
}

glu_status glu_add_rmsnorm_fwd(glu_dtype dtype, int64_t rows, int64_t hidden, const void *x, int64_t ldx,
                               const void *residual, int64_t ldr, const void *gamma, void *h, int64_t ldh,
                               void *y, int64_t ldy, float *rstd, float eps, hipStream_t stream)
{
    if (!(dtype >= GLU_F32 && dtype <= GLU_BF16))
        return GLU_ERR_ENUM;
    if (rows < 0 || hidden < 0)
        return GLU_ERR_SHAPE;
    if (!(eps > 0.0f) || !isfinite(eps))
        return GLU_ERR_ARG;
    if (rows == 0 || hidden == 0)
        return GLU_OK;
    if (rows > INT32_MAX || hidden > (int64_t(1) << 31))
        return GLU_ERR_SHAPE;
    if (x == nullptr || residual == nullptr || gamma == nullptr || h == nullptr || y == nullptr)
        return GLU_ERR_NULL;
    if (ldx < hidden || ldr < hidden || ldh < hidden || ldy < hidden)
        return GLU_ERR_STRIDE;
    const int es = glu::elem_size(dtype);
    const Region rx{uintptr_t(x), ldx, hidden}, rr{uintptr_t(residual), ldr, hidden};
    const Region rh{uintptr_t(h), ldh, hidden}, ry{uintptr_t(y), ldy, hidden};
    const Region rg{uintptr_t(gamma), hidden, hidden};
    int64_t ext;
    for (const Region *r : {&rx, &rr, &rh, &ry})
        if (!extent_bytes(rows, *r, es, &ext))
            return GLU_ERR_SHAPE;
    if (!extent_bytes(1, rg, es, &ext))
        return GLU_ERR_SHAPE;
    // outputs: exactly an input, or disjoint from every input; never each other
    const Region ins[2] = {rx, rr};
    if (bad_alias(rows, rh, ins, 2, es) || bad_alias(rows, ry, ins, 2, es))
        return GLU_ERR_ALIAS;
    if (overlaps(rows, rh, ry, es))
        return GLU_ERR_ALIAS;
    // gamma (one row) against the outputs: compare byte extents
    auto disjoint = [](uintptr_t a, int64_t na, uintptr_t b, int64_t nb) {
        return a + uintptr_t(na) <= b || b + uintptr_t(nb) <= a;
    };
    int64_t eh, ey;
    extent_bytes(rows, rh, es, &eh);
    extent_bytes(rows, ry, es, &ey);
    const int64_t eg = hidden * es;
    if (!disjoint(rg.p, eg, rh.p, eh) || !disjoint(rg.p, eg, ry.p, ey))
        return GLU_ERR_ALIAS;
    if (rstd != nullptr) {
        const uintptr_t rp = uintptr_t(rstd);
        const int64_t rn = rows * int64_t(sizeof(float));
        int64_t ex2, er2;
        extent_bytes(rows, rx, es, &ex2);
        extent_bytes(rows, rr, es, &er2);
        if (!disjoint(rp, rn, rx.p, ex2) || !disjoint(rp, rn, rr.p, er2) || !disjoint(rp, rn, rg.p, eg) ||
            !disjoint(rp, rn, rh.p, eh) || !disjoint(rp, rn, ry.p, ey))
            return GLU_ERR_ALIAS;
    }
    const Region all[5] = {rx, rr, rh, ry, rg};
    bool vec = true;
    for (const Region &r : all)
        if (!aligned16(r.p) || (rows > 1 && ((r.ld * es) & 15) != 0))
            vec = false;
    const glu::RmsShape shape = glu::rms_shape(hidden, vec ? glu::vec_elems(dtype) : 1);
    if (shape.vpt == 0 && (overlaps(rows, rh, rx, es) || overlaps(rows, rh, rr, es)))
        return GLU_ERR_ALIAS;   // the two-pass kernel re-reads x and residual
    glu::RmsArgs p{};
    p.x = x;
    p.res = residual;
    p.gamma = gamma;
    p.h = h;
    p.y = y;
    p.rstd = rstd;
    p.ldx = ldx;
    p.ldr = ldr;
    p.ldh = ldh;
    p.ldy = ldy;
    p.hidden = uint32_t(hidden);
    p.eps = eps;
    return glu::launch_add_rmsnorm(dtype, vec, shape, uint32_t(rows), p, stream) == hipSuccess ? GLU_OK
                                                                                                : GLU_ERR_HIP;
}

const char *glu_status_string(glu_status status)
{
    switch (status) {
    case GLU_OK: return "success";
    case GLU_ERR_NULL: return "a required pointer is NULL, or a pointer that must be NULL is not";
    case GLU_ERR_SHAPE: return "negative dimension, or the operand extent overflows";
    case GLU_ERR_STRIDE: return "a row stride is smaller than the row width";
    case GLU_ERR_ENUM: return "kind, layout or dtype out of range";
    case GLU_ERR_ALIAS: return "an output partially overlaps an input or another output";
    case GLU_ERR_INPLACE: return "inplace must be 0 or 1, and output pointers must be NULL when it is 1";
    case GLU_ERR_HIP: return "the HIP kernel launch failed";
    case GLU_ERR_ARG: return "a scalar argument is out of range (eps must be finite and > 0)";
    }
    return "unknown status";
}

int glu_version(void) { return (1 << 16) | 0; }

}  // extern "C"
