// ggrms_internal.h -- declarations shared by the host planner, the kernel
// tables and the launcher of libggrms.  Not installed; not part of the ABI.
#pragma once

#include <stdint.h>

#include "ggrms.h"
#include "ggrms_tuning.h"

namespace ggrms {

// Kernel arguments, passed by value.  Pointers already include the row
// offset of the launch chunk.  Strides are in elements.  Kept to 96 bytes:
// the HIP runtime enqueues a launch whose arguments fit in 96 bytes ~0.5 us
// faster than one with 128 or more (2.8 against 3.3-3.6 us of host time per
// launch, which is what a decode step's launches cost), so whatever the
// kernels can derive (units, the weight's stride between groups, the banded
// order's block sizes) is derived on the device, and the flags and shifts
// share one word.
//
// XCD-banded tile order (kBitBand; WAVE and BLOCK).  A tile is one
// workgroup's work: WAVE, threads / lanes consecutive groups of one row;
// BLOCK, one group of a row tile of UPB rows.  The launch's R x C tiles (R
// rows or row tiles, C = xc tile columns) are taken in blocks of 8 rows;
// inside a block, numbered column-major, XCD x takes the C tiles x*C ..
// x*C + C-1, i.e. a band of about C/8 columns of 8 rows.  Workgroups are dealt
// to the 8 XCDs in turn (workgroup b runs on XCD b % 8) and all XCDs move
// through the blocks at the same pace, so the tiles in flight still cover a
// contiguous run of rows -- the HBM access pattern of the row-major order --
// while each XCD reads the weights of only its band, which then stay in its
// L2 and its CUs' L1.  The last R % 8 rows form a short block, shared out the
// same way.
// With super-tiles of S = 2^kBitSuperShift tiles (WAVE tiles of packed
// groups, whose byte length is not a multiple of the 128-byte cache line), a
// full block is numbered by S consecutive tiles of one row at a time (super-
// tile (s, r) holds columns s*S .. s*S + S-1 of row r; super-tiles taken
// column-major), so the S tiles that share lines at their edges run on one
// XCD, one after the other, and each line is fetched into one L2 only.  The
// launch has C % S == 0; S = 1 is the plain banded order.
struct KArgs {
    const void* y;
    const void* gate;
    const float* w;
    void* out;
    int64_t sy, sg, so;
    uint32_t rows;    // rows in this launch
    uint32_t groups;  // groups per row
    uint32_t G;       // group size in elements
    uint32_t nvec;    // vectors per group; RUN: groups per run
    uint32_t div_m;   // magic multiplier for x / groups (RUN: x / runs per row; shift in bits)
    uint32_t xc;      // banded order: tile columns C (RUN: runs per row, either order)
    uint32_t xc_m;    // magic multiplier for x / C (shift in bits)
    float Ginv;       // 1/G rounded to f32 (the normaliser multiplies by it)
    float eps;
    uint32_t bits;    // kBit* fields below
};
static_assert(sizeof(KArgs) == 96, "kernel arguments must stay within 96 bytes");

// KArgs::bits
constexpr uint32_t kBitDivShift = 0;      // 5 bits: shift for x / groups
constexpr uint32_t kBitXcShift = 5;       // 5 bits: shift for x / C
constexpr uint32_t kBitRound = 1u << 10;  // round the intermediate (16-bit types only)
constexpr uint32_t kBitShared = 1u << 11; // one weight vector shared by every group
constexpr uint32_t kBitBand = 1u << 12;   // XCD-banded tile order
constexpr uint32_t kBitSuperShift = 13;   // 3 bits: log2 of the banded order's super-tile

// Workgroups are dealt to XCDs in turn on the 8-XCD part.
constexpr uint32_t kXcds = 8;

// Supported shapes.  WAVE: lanes in {1..64} (powers of two); vectors per lane
// 1 for lanes < 64 (also 2 with 8, 16 or 32 lanes for packed groups), 1..4
// for lanes == 64.  BLOCK: lanes in {128,256,512,1024},
// vectors per lane 1..4, and 6 with 256 lanes.  WIDE: 1024 lanes, vectors per
// lane 0 (it loops over the group).  RUN: 64 lanes, one or two vectors each,
// over a run of packed groups.  ROWS: 256 lanes x 3 vectors, or 320, 384, 448 or
// 512 lanes x 2 (16-byte vectors, not packed).  A WAVE workgroup is a single wave or 4
// waves (the kernel takes its size from the launch; the planner's rule says
// which).
constexpr int kWaveBlock = 256;
// Most groups one RUN wave takes (one lane per group forms the groups' sums).
constexpr int kRunMaxGroups = 32;
// A weight shared by every group is staged by the RUN wave, kRunStage floats
// per lane: groups of at most 512 elements (two of them fill the 128 slots).
constexpr int kRunStage = 8;
constexpr int kWaveBlockOneWave = 64;
constexpr int kWideBlock = 1024;
// ROWS: one workgroup per compute unit of the part (gfx950: 256), taken for
// jobs of at least kRowsMinUnits (row, group) units -- eight rows or more per
// workgroup, enough to amortise loading its weights and to keep rows in flight.
constexpr int64_t kRowsWorkgroups = 256;
constexpr int64_t kRowsMinUnits = 2048;

// Rows of one group per BLOCK workgroup (the workgroup stays <= 512 threads).
inline bool rows_per_workgroup_supported(int kernel, int lanes, int upb) {
    if (upb == 1) return true;
    if (kernel != GGRMS_KERNEL_BLOCK) return false;
    if (lanes == 128) return upb == 2 || upb == 4;
    if (lanes == 256) return upb == 2;
    return false;
}

inline bool shape_supported(int kernel, int lanes, int vpt) {
    switch (kernel) {
    case GGRMS_KERNEL_WAVE:  // (8, 16 or 32) x 2: packed groups only
        if (lanes == 64) return vpt >= 1 && vpt <= 4;
        if ((lanes == 8 || lanes == 16 || lanes == 32) && vpt == 2) return true;
        return (lanes == 1 || lanes == 2 || lanes == 4 || lanes == 8 || lanes == 16 ||
                lanes == 32) &&
               vpt == 1;
    case GGRMS_KERNEL_BLOCK:
        return (lanes == 128 || lanes == 256 || lanes == 512 || lanes == 1024) &&
               ((vpt >= 1 && vpt <= 4) || (lanes == 256 && vpt == 6));
    case GGRMS_KERNEL_WIDE:
        return lanes == kWideBlock;
    case GGRMS_KERNEL_RUN:
        return lanes == 64 && (vpt == 1 || vpt == 2);
    case GGRMS_KERNEL_ROWS:
        return (lanes == 256 && vpt == 3) ||
               ((lanes == 320 || lanes == 384 || lanes == 448 || lanes == 512 || lanes == 768 ||
                 lanes == 1024) &&
                vpt == 2);
    default:
        return false;
    }
}

// Full launch plan: the public plan plus what the launcher needs.
struct LaunchPlan {
    ggrms_plan_t pub;
    uint32_t flags;
    int esize;
    int64_t groups;
    int64_t nvec;
    int64_t rows_per_launch;  // rows handled by each launch (the last one may have fewer)
    bool xband;               // XCD-banded tile order (kBitBand)
    int super_shift;          // log2 of the banded order's super-tile (kBitSuperShift)
    int64_t runs_per_row;     // RUN: tiles of one row
    int64_t rows_stride;      // ROWS: workgroups per group, the step between a workgroup's rows
};

// WAVE: groups one workgroup covers (lanes <= 64).
inline int64_t wave_groups_per_workgroup(int lanes, int threads) { return threads / lanes; }

// Tile rows and tile columns of one launch over r rows (the banded order's R
// and C, described above KArgs); a WAVE tile is one workgroup.
inline void launch_tiles(const LaunchPlan& lp, int64_t r, int64_t* R, int64_t* C) {
    const ggrms_plan_t& p = lp.pub;
    if (p.kernel == GGRMS_KERNEL_BLOCK) {
        *R = (r + p.rows_per_workgroup - 1) / p.rows_per_workgroup;
        *C = lp.groups;
    } else if (p.kernel == GGRMS_KERNEL_WIDE) {  // one unit per workgroup, row-major only
        *R = r;
        *C = lp.groups;
    } else if (p.kernel == GGRMS_KERNEL_RUN) {  // one run per one-wave workgroup
        *R = r;
        *C = lp.runs_per_row;
    } else if (p.kernel == GGRMS_KERNEL_ROWS) {  // its own order (no banding)
        *R = r;
        *C = lp.groups;
    } else {
        const int64_t gpw = wave_groups_per_workgroup(p.lanes_per_group, p.block_threads);
        *R = r;
        *C = (lp.groups + gpw - 1) / gpw;
    }
}

// Workgroups of one launch over r rows.
inline int64_t launch_workgroups(const LaunchPlan& lp, int64_t r) {
    const ggrms_plan_t& p = lp.pub;
    switch (p.kernel) {
    case GGRMS_KERNEL_BLOCK:
        return (r + p.rows_per_workgroup - 1) / p.rows_per_workgroup * lp.groups;
    case GGRMS_KERNEL_WAVE: {
        if (lp.xband) {  // one workgroup per tile, tiles of one row
            int64_t R, C;
            launch_tiles(lp, r, &R, &C);
            return R * C;
        }
        const int64_t threads = r * lp.groups * p.lanes_per_group;  // units in a row-major run
        return (threads + p.block_threads - 1) / p.block_threads;
    }
    case GGRMS_KERNEL_WIDE: return r * lp.groups;
    case GGRMS_KERNEL_RUN: return r * lp.runs_per_row;
    case GGRMS_KERNEL_ROWS: return lp.rows_stride * lp.groups;
    default: return 0;
    }
}

// Operator flags the _ex calls take; the _tuned calls also take the
// ggrms_tuning_flag_t bits.
constexpr uint32_t kOperatorFlags =
    GGRMS_FLAG_ROUND_INTERMEDIATE | GGRMS_FLAG_NORM_BEFORE_GATE | GGRMS_FLAG_WEIGHT_PER_GROUP;
constexpr uint32_t kTuningFlags = GGRMS_FLAG_CACHE_STREAM | GGRMS_FLAG_CACHE_KEEP |
                                  GGRMS_FLAG_ORDER_ROWS | GGRMS_FLAG_ORDER_BANDED |
                                  GGRMS_FLAG_WAVE_ONE | GGRMS_FLAG_WAVE_FOUR;

// Validation and kernel choice; no HIP calls.  Implemented in plan.cpp.
// `flags` are ggrms_flag_t and ggrms_tuning_flag_t bits.  shape == nullptr
// picks everything; otherwise its vector_bytes (0 = widest allowed) must be
// allowed by the alignment, its lanes/vectors (both 0 = pick) must be built
// and cover the group (GGRMS_ERROR_NOT_SUPPORTED if not), and its
// rows_per_workgroup (0 = pick) must be built for the shape and allowed by
// the weight's alignment.
ggrms_status_t make_plan(const void* y, const void* gate, const float* w, const void* out,
                         int64_t rows, int64_t width, int64_t group_size, int64_t sy,
                         int64_t sg, int64_t so, float eps, int dtype, uint32_t flags,
                         const ggrms_shape_t* shape, LaunchPlan* plan);

// Magic numbers for n / d with n < 2^31 and 1 <= d < 2^31:
// q = (umulhi(n, m) + n) >> s.
void div_magic(uint32_t d, uint32_t* m, uint32_t* s);

// Kernel lookup per dtype (kernel tables); nullptr if the shape is not built.
// (nbg selects the norm-before-gate instantiations, in their own files; nt
// the variant whose y/gate/out accesses carry the non-temporal hint; pb the
// piece bytes: vb for group-aligned vectors, 2/4/8 for packed groups.)
const void* pick_f32(int kernel, int vb, int pb, int lanes, int vpt, int upb, bool nt);
const void* pick_f16(int kernel, int vb, int pb, int lanes, int vpt, int upb, bool nt);
const void* pick_bf16(int kernel, int vb, int pb, int lanes, int vpt, int upb, bool nt);
const void* pick_f32_nbg(int kernel, int vb, int pb, int lanes, int vpt, int upb, bool nt);
const void* pick_f16_nbg(int kernel, int vb, int pb, int lanes, int vpt, int upb, bool nt);
const void* pick_bf16_nbg(int kernel, int vb, int pb, int lanes, int vpt, int upb, bool nt);

}  // namespace ggrms
