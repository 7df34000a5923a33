// ggrms_internal.h -- declarations shared by the host planner, the kernel
// tables and the launcher of libggrms.  Not installed; not part of the ABI.
#pragma once

#include <stdint.h>

#include "ggrms.h"

namespace ggrms {

// Kernel arguments, passed by value.  Pointers already include the row
// offset of the launch chunk.  Strides are in elements.
struct KArgs {
    const void* y;
    const void* gate;
    const float* w;
    void* out;
    int64_t sy, sg, so;
    int64_t wgs;      // weight offset per group: G (one weight per column) or 0 (shared)
    uint32_t units;   // (row, group) units in this launch
    uint32_t rows;    // rows in this launch
    uint32_t groups;  // groups per row
    uint32_t div_m;   // magic multiplier for x / groups
    uint32_t div_s;   // shift for x / groups
    uint32_t G;       // group size in elements
    uint32_t nvec;    // vectors per group
    float Gf;         // (float)G
    float Ginv;       // 1/G rounded to f32 (the normaliser multiplies by it)
    float eps;
    int32_t ri;       // round the intermediate (16-bit types only)
};

// Supported shapes.  WAVE: lanes in {1..64} (powers of two); vectors per lane
// 1 for lanes < 64, 1..4 for lanes == 64.  BLOCK: lanes in {128,256,512,1024},
// vectors per lane 1..4.  WIDE: 1024 lanes, vectors per lane 0 (it loops over
// the group).  A WAVE workgroup is 256 threads (4 waves), or a single wave
// when every group shares one weight vector (the kernel takes its size from
// the launch): there a wave's slot is freed the moment it retires, instead
// of waiting for the slowest wave of its workgroup, which keeps more loads
// in flight -- 0.83 against 0.815 of HBM peak on 128-wide fp16 groups.  With
// a weight per column the 4-wave form is ahead (0.77 against 0.76).
constexpr int kWaveBlock = 256;
constexpr int kWaveBlockOneWave = 64;
constexpr int kWideBlock = 1024;

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
    case GGRMS_KERNEL_WAVE:
        if (lanes == 64) return vpt >= 1 && vpt <= 4;
        return (lanes == 1 || lanes == 2 || lanes == 4 || lanes == 8 || lanes == 16 ||
                lanes == 32) &&
               vpt == 1;
    case GGRMS_KERNEL_BLOCK:
        return (lanes == 128 || lanes == 256 || lanes == 512 || lanes == 1024) && vpt >= 1 &&
               vpt <= 4;
    case GGRMS_KERNEL_WIDE:
        return lanes == kWideBlock;
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
};

// Validation and kernel choice; no HIP calls.  Implemented in plan.cpp.
// `flags` are ggrms_flag_t bits.  shape == nullptr picks the shape; otherwise
// its lanes/vectors are used if built and covering the group
// (GGRMS_ERROR_NOT_SUPPORTED if not) and its rows_per_workgroup (0 = pick)
// must be built for the shape and allowed by the weight's alignment.
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
