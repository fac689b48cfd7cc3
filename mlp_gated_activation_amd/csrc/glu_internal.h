// glu_internal.h -- the launch plan passed from the host API (glu_api.cpp)
// to the kernels (glu_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace glu {

// Launch shape.  A "unit" is one 16-byte vector of every stream (8 bf16/fp16
// or 4 fp32 elements), or a single element on the unaligned path.  Each
// thread owns GLU_UNROLL units, BLOCK apart, so every wave's accesses to a
// stream are contiguous 1 KiB runs.  The defaults come from sweeps on
// MI355X (block 64..1024, unroll 1..8, with and without non-temporal hints,
// median of 3-5 interleaved rounds): many short-lived blocks with one vector
// per stream per thread moved the most bytes -- 64 threads for the forward
// (3 streams), 128 for the backward (5 streams).
#ifndef GLU_BLOCK
#define GLU_BLOCK 128
#endif
#ifndef GLU_BLOCK_FWD
#define GLU_BLOCK_FWD 64
#endif
#ifndef GLU_BLOCK_BWD
#define GLU_BLOCK_BWD GLU_BLOCK
#endif
// Backward launches of fewer than kCapMinUnits units (below 4096 x 8192
// bf16) finish in one or two rounds of workgroups, and there fewer, larger
// blocks start the streams sooner: bf16 SwiGLU backward, 4096 rows, 512
// against 128 threads (same process): 9.0 / 9.7 us at 1024 columns, 14.6 /
// 15.5 at 1792, 16.2 / 17.0 at 2048, 29.8 / 30.6 at 4096, 43.0 / 43.3 at 6144.
// From 4096 x 8192 up the capped 128-thread blocks are as fast or faster
// (4096 x 11008: 73.3 / 72.4 us; 4096 x 14336: 94.1 / 93.4).  The forward
// keeps 64 threads at every size (1024 columns: even with 256..1024).
#ifndef GLU_BLOCK_BWD_SMALL
#define GLU_BLOCK_BWD_SMALL 512
#endif
#ifndef GLU_UNROLL
#define GLU_UNROLL 1
#endif
// 1: 16-byte loads / stores carry the non-temporal hint (streamed, not kept).
#ifndef GLU_NT
#define GLU_NT 1
#endif
#ifndef GLU_NT_LOAD
#define GLU_NT_LOAD GLU_NT
#endif
#ifndef GLU_NT_STORE
#define GLU_NT_STORE GLU_NT
#endif
// 1: sigmoids of bf16/fp16 data use the raw hardware exp on a 2^16-scaled
// argument (2 instructions) instead of the subnormal-safe exp2f (7).
#ifndef GLU_SCALED_EXP
#define GLU_SCALED_EXP 1
#endif
// 1: remap block ids so each of the 8 XCDs walks one contiguous slice.
#ifndef GLU_XCD_REMAP
#define GLU_XCD_REMAP 0
#endif

// LDS reserved per workgroup (never accessed) to cap the workgroups resident
// on a CU, 160 KiB of LDS each: 25 forward (64 threads), 10 backward (128
// threads).  Applied to 16-bit data in launches of at least kCapMinUnits
// units; the launcher in glu_kernels.hip gives the measurements.
constexpr unsigned kCapLdsFwd = 6400, kCapLdsBwd = 16384;
#ifndef GLU_CAP_MIN_UNITS
#define GLU_CAP_MIN_UNITS (1u << 22)
#endif
constexpr uint32_t kCapMinUnits = GLU_CAP_MIN_UNITS;

// Largest unit count one launch covers; keeps every per-launch index below
// 2^31, which the kernels' 32-bit unsigned division relies on.
constexpr uint32_t kMaxUnitsPerLaunch = 1u << 30;
// Widest row (in elements) one launch covers: column indices stay 32-bit
// with room for one more vector.  Longer rows are split into column chunks.
constexpr int64_t kMaxColsPerLaunch = int64_t(1) << 31;

// Division by a runtime constant d >= 1 for numerators n < 2^31:
//   n / d == (umulhi(n, magic) + n) >> shift
// with shift = ceil(log2 d) and magic = floor(2^32 * (2^shift - d) / d) + 1.
struct Divider {
    uint32_t magic;
    uint32_t shift;
};

inline Divider make_divider(uint32_t d)
{
    uint32_t s = 0;
    while (s < 32 && (uint64_t(1) << s) < d)
        ++s;
    uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1;
    return Divider{uint32_t(m), s};
}

// Kernel arguments: one plan per launch.  Pointers are byte addresses of
// element (0, 0) of each operand; row strides are in elements.
struct Args {
    const void *in0;   // a
    const void *in1;   // b
    const void *in2;   // dy (backward only)
    void *out0;        // y (forward) or da (backward)
    void *out1;        // db (backward only)
    int64_t ld_in0, ld_in1, ld_in2, ld_out0, ld_out1;
    uint32_t units;          // units in this launch (< 2^31)
    uint32_t units_per_row;  // ceil(cols / elements per unit)
    uint32_t cols;           // elements per row in this launch
    Divider row_div;         // division by units_per_row
};

enum Dtype { F32 = 0, F16 = 1, BF16 = 2 };


// Strided operands of any layout, processed in 64 x 64 tiles staged through
// LDS: every operand is read or written along its own contiguous direction.
constexpr int kTile = 64;
// How a tiled-kernel operand moves between HBM and registers.
enum TileMode : uint8_t {
    kDirect = 0,      // column stride 1, 16-byte aligned: 16-byte chunks along the row
    kTransposed = 1,  // row stride 1, 16-byte aligned: 16-byte chunks down the column, through LDS
    kGather = 2,      // anything else (broadcast, sliced, unaligned): element by element
};

struct TileArgs {
    const void *in[3];      // a, b, dy
    void *out[2];           // y | da, db
    int64_t irs[3], ics[3]; // input row / column strides (elements)
    int64_t ors[2], ocs[2];
    int64_t rows, cols;
    uint32_t tiles_r, tiles_c;
    uint32_t tile0;         // first tile (in launch order) of this launch
    uint8_t in_mode[3];     // TileMode per operand
    uint8_t out_mode[2];
    uint8_t in_slot[3];     // LDS slot of each kTransposed operand
    uint8_t out_slot[2];
    uint8_t nslots;         // slots the launch allocates: max(transposed inputs, transposed outputs)
};

#ifndef GLU_TILE_GROUP
#define GLU_TILE_GROUP 8
#endif
constexpr uint32_t kTileGroup = GLU_TILE_GROUP;

#if defined(__HIPCC__)
#define GLU_HD __host__ __device__
#else
#define GLU_HD
#endif

// Launch order of the tiles: bands of kTileGroup tile rows, walked column
// by column inside a band.  The blocks in flight then cover a strip of
// kTileGroup*64 rows, so row-major operands are read in long runs along
// each row and column-major ones in runs of kTileGroup*64 elements down each
// column.  Tile t of the order covers rows [64*r, 64*r + 64) and columns
// [64*c, 64*c + 64).
struct TileCoord {
    uint32_t r, c;
};
GLU_HD inline TileCoord grouped_coord(uint32_t t, uint32_t tiles_r, uint32_t tiles_c, uint32_t group)
{
    const uint64_t per_group = uint64_t(group) * tiles_c;
    const uint32_t g = uint32_t(t / per_group);
    const uint32_t first = g * group;
    const uint32_t h = tiles_r - first < group ? tiles_r - first : group;
    const uint64_t in_g = t - uint64_t(g) * per_group;
    return TileCoord{first + uint32_t(in_g % h), uint32_t(in_g / h)};
}
GLU_HD inline TileCoord tile_coord(uint32_t t, uint32_t tiles_r, uint32_t tiles_c)
{
    return grouped_coord(t, tiles_r, tiles_c, kTileGroup);
}

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2.  xcd_remap gives XCD x a contiguous range of the launch order, so the
// workgroups that run together on one XCD work on neighbouring tiles.  It is
// a bijection on [0, n) for any n.
constexpr uint32_t kXcds = 8;
GLU_HD inline uint32_t xcd_remap(uint32_t b, uint32_t n)
{
    const uint32_t q = n / kXcds, r = n % kXcds, x = b % kXcds;
    return x * q + (x < r ? x : r) + b / kXcds;
}

// Largest tile count one launch covers.
// grid * 256 threads must stay below 2^32 work-items per dimension
constexpr uint32_t kMaxTilesPerLaunch = 1u << 22;

hipError_t launch_tiles(int dtype, int kind, bool backward, const TileArgs &args, uint32_t ntiles,
                        hipStream_t stream);

// Enqueues one launch; returns the HIP status of hipLaunchKernel.
hipError_t launch(int dtype, int kind, bool backward, bool vec, const Args &args,
                  hipStream_t stream);

// Elements moved per unit on the vector path, by dtype.
inline int vec_elems(int dtype) { return dtype == F32 ? 4 : 8; }
inline int elem_size(int dtype) { return dtype == F32 ? 4 : 2; }

}  // namespace glu
