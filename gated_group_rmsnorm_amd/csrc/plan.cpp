// plan.cpp -- argument checks and kernel choice for ggrms_forward / ggrms_plan.
// Pure host C++: no HIP call happens here, so every error path can be
// exercised on a machine without a GPU.
#include <stdint.h>
#include <string.h>

#include <cmath>

#include "ggrms_internal.h"

namespace ggrms {
namespace {

bool mul_add_ok(int64_t a, int64_t b, int64_t c, int64_t* r) {
    int64_t m;
    if (__builtin_mul_overflow(a, b, &m)) return false;
    return !__builtin_add_overflow(m, c, r);
}

// Byte extent of a [rows, width] view: (rows-1)*stride + width elements.
bool extent_bytes(int64_t rows, int64_t width, int64_t stride, int esize, int64_t* bytes) {
    int64_t elems;
    if (!mul_add_ok(rows - 1, rows > 1 ? stride : 0, width, &elems)) return false;
    if (__builtin_mul_overflow(elems, (int64_t)esize, bytes)) return false;
    return true;
}

// Whether two [rows, width] views with byte row strides sa, sb and a row
// length of len bytes share any element.  Exact for equal strides; for
// unequal strides any overlap of the address ranges counts.
bool views_overlap(uintptr_t a, int64_t sa, uintptr_t b, int64_t sb, int64_t rows, int64_t len,
                   int64_t ext_a, int64_t ext_b) {
    // address ranges [a, a+ext_a) and [b, b+ext_b)
    if (a + (uintptr_t)ext_a <= b || b + (uintptr_t)ext_b <= a) return false;
    if (rows == 1 || sa != sb) return true;
    // element (i, c) of A meets element (j, d) of B iff (i-j)*s = D + d - c
    // for |d - c| < len, i.e. some k in [-(rows-1), rows-1] has |k*s - D| < len.
    const int64_t s = sa;
    const int64_t D = (int64_t)(b - a);  // wraps correctly for b < a
    int64_t k0 = D / s;                  // truncates toward zero
    for (int64_t k = k0 - 1; k <= k0 + 1; ++k) {
        if (k < -(rows - 1) || k > rows - 1) continue;
        const int64_t diff = k * s - D;
        if (diff < len && diff > -len) return true;
    }
    return false;
}

// Whether a [rows, len-byte] view at a with byte row stride sa (>= len when
// rows > 1) shares any byte with the range [b, b + nb).  Exact: row i covers
// [a + i*sa, a + i*sa + len), and some row meets the range iff an integer i in
// [0, rows) has b - a - len < i*sa < b + nb - a.
bool view_meets_range(uintptr_t a, int64_t sa, int64_t rows, int64_t len, int64_t ext_a,
                      uintptr_t b, int64_t nb) {
    if (a + (uintptr_t)ext_a <= b || b + (uintptr_t)nb <= a) return false;
    if (rows == 1) return true;
    const int64_t D = (int64_t)(b - a);  // |D| < 2^63: both ranges fit the address space
    // smallest i with i*sa > D - len, largest i with i*sa < D + nb
    const int64_t lo = D - len;
    int64_t i0 = lo >= 0 ? lo / sa + 1 : -((-lo) / sa);
    const int64_t hi = D + nb;
    int64_t i1 = hi > 0 ? (hi - 1) / sa : -((-hi) / sa) - 1;
    if (i0 < 0) i0 = 0;
    if (i1 > rows - 1) i1 = rows - 1;
    return i0 <= i1;
}

int64_t round_up_pow2(int64_t x) {
    int64_t p = 1;
    while (p < x) p <<= 1;
    return p;
}

// Largest packed group, in 16-byte vectors (512 lanes x 4 vectors); wider
// groups keep the narrower vectors.
constexpr int64_t kMaxPackedVectors = 2048;

// Most vectors of a group for which the library takes ROWS itself (it can
// be forced up to 2048).
constexpr int64_t kRowsMaxDefaultVectors = 1792;

// Waves of a job that the part holds at once with room to spare (256 CUs x 4
// SIMDs x 4 waves): such a job is a single round of loads and arithmetic.
constexpr int64_t kSmallJobWaves = 4096;

// ROWS shape for a group of nvec 16-byte vectors (nvec <= 2048): 256 lanes x
// 3 up to 608 vectors, above that two vectors on the next multiple of 64
// lanes up to 1024 vectors -- the fastest of the built shapes in a sweep of
// 377 MB single-group bf16 jobs over groups of 528-1024 vectors (0.77-0.81 of
// HBM peak against 0.74-0.77 for the BLOCK kernel's one row per workgroup;
// 320 x 2 on the 5120-wide group: 58.6 against 63.0 us) -- and 768 or 1024
// lanes x 2 for 1025-2048 vectors.
void rows_shape(int64_t nvec, int* lanes, int* vpt) {
    if (nvec <= 608) {
        *lanes = 256;
        *vpt = 3;
    } else if (nvec <= 1024) {
        *lanes = (int)((nvec + 127) / 128 * 64);
        *vpt = 2;
    } else {
        *lanes = nvec <= 1536 ? 768 : 1024;
        *vpt = 2;
    }
}

int kernel_for_shape(int lanes, int vpt) {
    if (vpt == 0) return GGRMS_KERNEL_WIDE;
    return lanes <= 64 ? GGRMS_KERNEL_WAVE : GGRMS_KERNEL_BLOCK;
}

// Kernel shape for a group of nvec vectors, and the rows of one group a
// BLOCK workgroup takes (1 means no weight staging).  The table comes from
// sweeps of every built shape on gfx950 at ~377 MB per launch (bf16 jobs over
// group widths 8..32768, plus fp16 and f32 spot checks), timed after the
// clocks settle:
//   * up to 64 vectors: one vector per lane, the smallest power-of-two lane
//     segment, several groups per wave (WAVE kernel, 80-83% of HBM peak);
//   * 65-80: one wave, two vectors per lane (67-77%; 128 lanes: 64-75%);
//   * 81-96: two waves, one vector per lane, one row per workgroup (79-80%);
//   * 97-512: 128 or 256 lanes with 1-3 vectors each and 2-4 rows per
//     workgroup sharing staged weights (73-82%): 4 rows for 105-128 and
//     145-192 vectors, 2 elsewhere (1-2% apart at the band edges); never 4
//     at three vectors per lane, where the staging registers cost occupancy;
//   * 513-768: 256 lanes x 3 vectors, one row per workgroup (75-76%; 2 rows:
//     72-75%);
//   * 769-4096: 256-1024 lanes x 3-6 vectors, one row per workgroup (staging
//     at 4 vectors per lane measured 46-59% against 77% without); fewer waves
//     with more vectors each where the registers allow (1025-1536: 256 x 6,
//     0.75 against 0.67-0.71 for 512 x 3; 6 vectors take 163 VGPRs, 8 took
//     218 and lost to 512 x 4 and 1024 x 4);
//   * wider groups loop over the row twice (WIDE).
// In jobs of 2048 (row, group) units or more, groups of 513-1792 vectors take
// the ROWS kernel instead (rows_shape).
struct ShapeRule {
    int64_t max_nvec;
    int kernel, lanes, vpt, upb;
};
const ShapeRule kRules[] = {
    {80, GGRMS_KERNEL_WAVE, 64, 2, 1},
    {96, GGRMS_KERNEL_BLOCK, 128, 1, 1},
    {104, GGRMS_KERNEL_BLOCK, 128, 1, 2},
    {128, GGRMS_KERNEL_BLOCK, 128, 1, 4},
    {144, GGRMS_KERNEL_BLOCK, 128, 2, 2},
    {192, GGRMS_KERNEL_BLOCK, 128, 2, 4},
    {256, GGRMS_KERNEL_BLOCK, 256, 1, 2},
    {384, GGRMS_KERNEL_BLOCK, 128, 3, 2},
    {512, GGRMS_KERNEL_BLOCK, 256, 2, 2},
    {768, GGRMS_KERNEL_BLOCK, 256, 3, 1},
    {1024, GGRMS_KERNEL_BLOCK, 256, 4, 1},
    {1536, GGRMS_KERNEL_BLOCK, 256, 6, 1},
    {2048, GGRMS_KERNEL_BLOCK, 512, 4, 1},
    {3072, GGRMS_KERNEL_BLOCK, 1024, 3, 1},
    {4096, GGRMS_KERNEL_BLOCK, 1024, 4, 1},
};

// RUN length for packed groups of gbytes bytes (pb = gcd(gbytes, 16)): the
// groups per wave and, unless forced (force_vpt 1 or 2), the vectors per lane.
// A run of a multiple of 16 / pb groups spans a whole number of vectors, so
// every run of the row starts on a vector boundary and is stored in whole
// vectors; another run takes up to ceil((16 - pb + gpw * gbytes) / 16)
// vectors and shares a boundary vector with each neighbour.  Taken: the run
// that fills the most of its 64 x vpt slots, an aligned run counting 0.1
// more, two vectors per lane on a tie.  At most kRunMaxGroups groups.
int64_t run_length(int64_t gbytes, int pb, int force_vpt, int* vpt_out) {
    const int64_t k0 = 16 / pb;
    double best = -1.0;
    int64_t best_gpw = 0;
    int best_vpt = 0;
    for (int vpt = 2; vpt >= 1; --vpt) {
        if (force_vpt && vpt != force_vpt) continue;
        const int64_t cap = 64 * 16 * (int64_t)vpt;  // bytes the slots hold
        int64_t ga = cap / gbytes;
        if (ga > kRunMaxGroups) ga = kRunMaxGroups;
        ga = ga / k0 * k0;
        int64_t gm = (cap - 16 + pb) / gbytes;
        if (gm > kRunMaxGroups) gm = kRunMaxGroups;
        const double fa = ga >= 2 ? (double)(ga * gbytes) / (double)cap + 0.1 : -1.0;
        const double fm = gm >= 2 ? (double)(gm * gbytes) / (double)cap : -1.0;
        const int64_t g = fa >= fm ? ga : gm;
        const double f = fa >= fm ? fa : fm;
        if (f > best + 1e-9) {
            best = f;
            best_gpw = g;
            best_vpt = vpt;
        }
    }
    *vpt_out = best_vpt;
    return best > 0.0 ? best_gpw : 0;
}

void choose_shape(int64_t nvec, int* kernel, int* lanes, int* vpt, int* upb) {
    if (nvec <= 64) {
        *kernel = GGRMS_KERNEL_WAVE;
        *lanes = (int)round_up_pow2(nvec);
        *vpt = 1;
        *upb = 1;
        return;
    }
    for (const ShapeRule& r : kRules) {
        if (nvec <= r.max_nvec) {
            *kernel = r.kernel;
            *lanes = r.lanes;
            *vpt = r.vpt;
            *upb = r.upb;
            return;
        }
    }
    *kernel = GGRMS_KERNEL_WIDE;
    *lanes = kWideBlock;
    *vpt = 0;
    *upb = 1;
}

}  // namespace

void div_magic(uint32_t d, uint32_t* m, uint32_t* s) {
    // Round-up method of Granlund and Montgomery ("Division by invariant
    // integers using multiplication", PLDI 1994): l = ceil(log2 d),
    // m = floor(2^32 (2^l - d) / d) + 1; for n < 2^31, n / d = (mulhi(m, n) + n) >> l.
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    const uint64_t mm = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
    *m = (uint32_t)mm;
    *s = l;
}

ggrms_status_t make_plan(const void* y, const void* gate, const float* w, const void* out,
                         int64_t rows, int64_t width, int64_t group_size, int64_t sy,
                         int64_t sg, int64_t so, float eps, int dtype, uint32_t flags,
                         const ggrms_shape_t* shape, LaunchPlan* plan) {
    if (!plan) return GGRMS_ERROR_INVALID_VALUE;
    memset(plan, 0, sizeof *plan);
    if (rows < 0 || width <= 0 || group_size <= 0 || width % group_size != 0)
        return GGRMS_ERROR_INVALID_VALUE;
    if (flags & ~(kOperatorFlags | kTuningFlags)) return GGRMS_ERROR_INVALID_VALUE;
    if (shape && (shape->lanes_per_group < 0 || shape->vectors_per_lane < 0 ||
                  shape->rows_per_workgroup < 0 ||
                  (shape->vector_bytes != 0 && shape->vector_bytes != 2 &&
                   shape->vector_bytes != 4 && shape->vector_bytes != 8 &&
                   shape->vector_bytes != 16) ||
                  (shape->kernel != 0 && shape->kernel != GGRMS_KERNEL_RUN &&
                   shape->kernel != GGRMS_KERNEL_ROWS)))
        return GGRMS_ERROR_INVALID_VALUE;
    if (((flags & GGRMS_FLAG_ORDER_ROWS) && (flags & GGRMS_FLAG_ORDER_BANDED)) ||
        ((flags & GGRMS_FLAG_WAVE_ONE) && (flags & GGRMS_FLAG_WAVE_FOUR)))
        return GGRMS_ERROR_INVALID_VALUE;
    if ((flags & GGRMS_FLAG_ROUND_INTERMEDIATE) && (flags & GGRMS_FLAG_NORM_BEFORE_GATE))
        return GGRMS_ERROR_INVALID_VALUE;
    if ((flags & GGRMS_FLAG_CACHE_STREAM) && (flags & GGRMS_FLAG_CACHE_KEEP))
        return GGRMS_ERROR_INVALID_VALUE;
    plan->flags = flags;
    const int64_t wlen = (flags & GGRMS_FLAG_WEIGHT_PER_GROUP) ? group_size : width;
    if (!std::isfinite(eps) || eps < 0.0f) return GGRMS_ERROR_INVALID_VALUE;
    if (dtype != GGRMS_F32 && dtype != GGRMS_F16 && dtype != GGRMS_BF16)
        return GGRMS_ERROR_NOT_SUPPORTED;
    const int esize = dtype == GGRMS_F32 ? 4 : 2;
    plan->esize = esize;
    plan->groups = width / group_size;
    if (rows == 0) {
        plan->pub.kernel = GGRMS_KERNEL_NONE;
        return GGRMS_SUCCESS;
    }
    if (!y || !gate || !w || !out) return GGRMS_ERROR_INVALID_VALUE;
    if (rows > 1 && (sy < width || sg < width || so < width)) return GGRMS_ERROR_INVALID_VALUE;
    const uintptr_t py = (uintptr_t)y, pg = (uintptr_t)gate, po = (uintptr_t)out,
                    pw = (uintptr_t)w;
    if (py % esize || pg % esize || po % esize || pw % 4) return GGRMS_ERROR_INVALID_VALUE;
    if (rows == 1) sy = sg = so = width;  // strides of a single row are never used
    int64_t ey, eg, eo, ew, row_bytes;
    if (!extent_bytes(rows, width, sy, esize, &ey) || !extent_bytes(rows, width, sg, esize, &eg) ||
        !extent_bytes(rows, width, so, esize, &eo) || __builtin_mul_overflow(wlen, (int64_t)4, &ew) ||
        __builtin_mul_overflow(width, (int64_t)esize, &row_bytes))
        return GGRMS_ERROR_INVALID_VALUE;
    if (py + (uintptr_t)ey < py || pg + (uintptr_t)eg < pg || po + (uintptr_t)eo < po ||
        pw + (uintptr_t)ew < pw)
        return GGRMS_ERROR_INVALID_VALUE;
    // out may be y or gate exactly (in place); any other shared element is an error.
    const int64_t by = sy * esize, bg = sg * esize, bo = so * esize;
    const bool alias_y = po == py && bo == by;
    const bool alias_g = po == pg && bo == bg;
    if (!alias_y && views_overlap(po, bo, py, by, rows, row_bytes, eo, ey))
        return GGRMS_ERROR_INVALID_VALUE;
    if (!alias_g && views_overlap(po, bo, pg, bg, rows, row_bytes, eo, eg))
        return GGRMS_ERROR_INVALID_VALUE;
    // Every row reads the weight, so out must not share a byte with it.
    if (view_meets_range(po, bo, rows, row_bytes, eo, pw, ew)) return GGRMS_ERROR_INVALID_VALUE;

    // Widest vector every access can use: the three views' base pointers and
    // row strides, the group's byte length, and the matching weight loads
    // (or the caller's vector width, if those allow it).
    auto vector_fits = [&](int cand) {
        const int64_t wal = cand / esize * 4 < 16 ? cand / esize * 4 : 16;
        return py % cand == 0 && pg % cand == 0 && po % cand == 0 && by % cand == 0 &&
               bg % cand == 0 && bo % cand == 0 && (group_size * esize) % cand == 0 &&
               pw % wal == 0;
    };
    const int force_vb = shape ? shape->vector_bytes : 0;
    if (force_vb && force_vb < esize) return GGRMS_ERROR_NOT_SUPPORTED;
    int vb = esize;
    for (int cand = 16; cand > esize; cand >>= 1) {
        if (vector_fits(cand) && (!force_vb || cand == force_vb)) {
            vb = cand;
            break;
        }
    }
    int64_t nvec = group_size * esize / vb;
    int pb = vb;
    // Packed groups: the group's byte length is not a multiple of 16 but the
    // rows are 16-byte aligned and a multiple of 16 bytes long, so 16-byte
    // vectors counted from the row start never leave the row.  A unit takes
    // the vectors holding any of its elements -- at most
    // ceil((16 - pb + group bytes) / 16), since group starts fall on
    // multiples of pb = gcd(group bytes, 16) -- and stores boundary vectors in
    // pb-byte pieces.  For groups of more than one vector.  A per-column
    // weight must be 16-byte aligned (its vectors then line up with the
    // data's); one [G] weight shared by every group is read piece by piece
    // (a packed vector's weights wrap around the shared vector), each piece's
    // pb / esize weights in one load, so it must be aligned to that many
    // floats.
    const int64_t gbytes = group_size * esize;
    const bool shared_w = (flags & GGRMS_FLAG_WEIGHT_PER_GROUP) != 0;
    int64_t gcd = 16;
    while (gbytes % gcd) gcd >>= 1;
    if (vb < 16 && (!force_vb || force_vb == 16) && gbytes > 16 && row_bytes % 16 == 0 &&
        py % 16 == 0 && pg % 16 == 0 &&
        po % 16 == 0 && by % 16 == 0 && bg % 16 == 0 && bo % 16 == 0 &&
        pw % (shared_w ? 4 * gcd / esize : 16) == 0) {
        const int64_t nvp = (16 - gcd + gbytes + 15) / 16;
        if (nvp <= kMaxPackedVectors) {
            vb = 16;
            pb = (int)gcd;
            nvec = nvp;
        }
    }
    if (force_vb && vb != force_vb) return GGRMS_ERROR_NOT_SUPPORTED;
    const bool packed = pb < vb;
    int kernel = 0, lanes = 0, vpt = 0, rule_upb = 1;
    const int force_upb = shape ? shape->rows_per_workgroup : 0;
    // RUN: a wave takes gpw consecutive packed groups of a row on run_vpt
    // vectors per lane (forced: the shape's, if it gives one).
    const int force_run_vpt =
        shape && shape->kernel == GGRMS_KERNEL_RUN ? shape->vectors_per_lane : 0;
    int run_vpt = 0;
    const int64_t gpw = packed ? run_length(gbytes, pb, force_run_vpt, &run_vpt) : 0;
    // (a weight shared by every group is staged in LDS by the run's wave:
    // groups of at most 64 x kRunStage elements)
    const bool run_fits = packed && gpw >= 2 &&
                          (!(flags & GGRMS_FLAG_WEIGHT_PER_GROUP) || group_size <= 64 * kRunStage);
    // ROWS needs 16-byte vectors that are not packed and a launch of
    // 32-bit row indices
    const bool rows_fit = !packed && vb == 16 && rows < ((int64_t)1 << 31) && nvec <= 2048;
    if (shape && shape->kernel == GGRMS_KERNEL_ROWS) {
        if (!rows_fit || force_upb > 1) return GGRMS_ERROR_NOT_SUPPORTED;
        if (shape->lanes_per_group == 0 && shape->vectors_per_lane == 0) {
            rows_shape(nvec, &lanes, &vpt);
        } else {
            lanes = shape->lanes_per_group;
            vpt = shape->vectors_per_lane;
        }
        if (!shape_supported(GGRMS_KERNEL_ROWS, lanes, vpt) || (int64_t)lanes * vpt < nvec)
            return GGRMS_ERROR_NOT_SUPPORTED;
        kernel = GGRMS_KERNEL_ROWS;
    } else if (shape && shape->kernel == GGRMS_KERNEL_RUN) {
        if (!run_fits || !(shape->lanes_per_group == 0 || shape->lanes_per_group == 64) ||
            !(shape->vectors_per_lane == 0 || shape_supported(GGRMS_KERNEL_RUN, 64,
                                                              shape->vectors_per_lane)) ||
            force_upb > 1)
            return GGRMS_ERROR_NOT_SUPPORTED;
        kernel = GGRMS_KERNEL_RUN;
        lanes = 64;
        vpt = run_vpt;
    } else if (shape && (shape->lanes_per_group != 0 || shape->vectors_per_lane != 0)) {
        kernel = kernel_for_shape(shape->lanes_per_group, shape->vectors_per_lane);
        lanes = shape->lanes_per_group;
        vpt = shape->vectors_per_lane;
        if (!shape_supported(kernel, lanes, vpt)) return GGRMS_ERROR_NOT_SUPPORTED;
        if (kernel != GGRMS_KERNEL_WIDE && (int64_t)lanes * vpt < nvec)
            return GGRMS_ERROR_NOT_SUPPORTED;
        rule_upb = rows_per_workgroup_supported(kernel, lanes, 4) ? 4
                   : rows_per_workgroup_supported(kernel, lanes, 2) ? 2 : 1;
        if (vpt > 1 && rule_upb > 2) rule_upb = 2;
        if (vpt > 2) rule_upb = 1;
    } else {
        choose_shape(nvec, &kernel, &lanes, &vpt, &rule_upb);
        // Packed groups keep one vector per lane on their lane segment, with
        // the boundary vectors inside a wave merged, in small jobs too: half
        // the lanes with two vectors each (the same slots, each wave's fixed
        // work over twice the elements) stores every boundary vector in
        // pieces, and lost on two machines for the strided 256 x 4800 fp16 job
        // (4.17 and 3.96 us against 3.90 and 3.67 for 16 x 1; with the
        // two-vector boundaries merged too, 4.45 and 4.43).  Jobs resident at
        // once (at most kSmallJobWaves waves) do not take runs either.
        const bool small_job = rows * plan->groups * lanes <= kSmallJobWaves * 64;
        if (packed && kernel == GGRMS_KERNEL_WAVE && !small_job && run_fits && lanes < 64 &&
            2 * gpw * gbytes >= 64 * 16 * run_vpt && 10 * gbytes < 6 * 16 * lanes && vpt == 1) {
            // Larger jobs of packed groups that fill less than 60% of their
            // lane segment (groups just over a power of two of vectors, or
            // a few vectors): runs of groups per wave over a contiguous
            // stretch of the row, as long as the run fills at least half of
            // its slots.  377 MB of 127-wide bf16 groups (15.9 vectors on 32
            // lanes): 70.4 us in runs of 8 with two vectors per lane (every
            // run on a vector boundary), against 86-88 for runs of 3 with one
            // vector per lane and 93.4 for the segments; 13-wide fp16 groups
            // (3.25 vectors on 4 lanes): 62 us in runs of 32.  Fuller
            // segments stay ahead (same machine; runs with one and with two
            // vectors per lane): 100-wide fp16 63.3 against 71.2 / 69.5 us,
            // 99-wide bf16 72.0 against 74.7 / 78.4, 50-wide bf16 67.7
            // against 73.6 / 78.0, 25-wide f32 65.0 against 71.6 / 73.1 --
            // except 250-wide fp16 (31.3 vectors on 32 lanes), where runs of
            // 4 on two vectors per lane were 4% ahead (66.4 against 69.6).
            // Groups of 33-38 vectors (64-lane segments under 60% full) stay
            // on their segments too: 300-wide fp16 66.7 against 76.5 us for
            // runs of 3 on two vectors per lane, 290-wide 73.7 against 78.2.
            kernel = GGRMS_KERNEL_RUN;
            lanes = 64;
            vpt = run_vpt;
        } else if (kernel == GGRMS_KERNEL_BLOCK && rows_fit && nvec > 512 &&
                   nvec <= kRowsMaxDefaultVectors && plan->groups <= kRowsWorkgroups &&
                   rows * plan->groups >= kRowsMinUnits) {
            // Wide groups in large jobs: one workgroup per compute unit
            // taking rows in turn, with the next rows' inputs in flight
            // while it stores, instead of one workgroup per row (whose
            // loads start only when a slot frees).  Groups of 1025-1792
            // vectors on 768 or 1024 lanes x 2, 377 MB bf16 jobs against
            // the BLOCK shapes with one row per workgroup: 9216 wide 62.8
            // against 64.8 us, 10240 61.9 / 63.4, 12288 61.8 / 62.5, 14336
            // 64.2 / 68.2; at 16384 (2048 vectors) BLOCK 512 x 4 stays
            // ahead, 63.7 against 64.2.
            kernel = GGRMS_KERNEL_ROWS;
            rows_shape(nvec, &lanes, &vpt);
        }
    }
    if (kernel == GGRMS_KERNEL_RUN) {
        plan->runs_per_row = (plan->groups + gpw - 1) / gpw;
        plan->pub.groups_per_run = (int32_t)gpw;
        nvec = gpw;  // the kernel takes the run length in the vector-count field
    }
    if (packed && kernel == GGRMS_KERNEL_WIDE) return GGRMS_ERROR_NOT_SUPPORTED;  // not built
    // two vectors per lane below 64 lanes: built for packed groups only
    if (!packed && kernel == GGRMS_KERNEL_WAVE && lanes < 64 && vpt > 1)
        return GGRMS_ERROR_NOT_SUPPORTED;

    const int64_t groups = plan->groups;
    // Rows of one group per BLOCK workgroup: the group's weights are staged
    // once in LDS with 16-byte loads, so the weight must be 16-byte aligned
    // and the group a multiple of 4 floats; no more rows than the job has.
    const bool can_stage = pw % 16 == 0 && group_size % 4 == 0 && !packed;
    int upb = 1;
    if (force_upb) {
        if (!rows_per_workgroup_supported(kernel, lanes, force_upb) ||
            (force_upb > 1 && !can_stage))
            return GGRMS_ERROR_NOT_SUPPORTED;
        upb = force_upb;
    } else if (can_stage) {
        upb = rule_upb;
        while (upb > 1 && (rows < upb || !rows_per_workgroup_supported(kernel, lanes, upb)))
            upb >>= 1;
    }
    plan->pub.kernel = kernel;
    plan->pub.lanes_per_group = lanes;
    plan->pub.rows_per_workgroup = upb;
    // WAVE workgroups: one wave for 16-byte vectors, packed groups included,
    // whose slot is freed the moment it retires (128-wide groups: 0.83
    // against 0.79 of HBM peak with four; 377 MB of 100-wide packed fp16
    // groups: 62.7 against 67.7 us; the strided 256 x 4800 fp16 job: equal
    // with 16 x 1, before the boundary merge); four waves for narrower
    // vectors, which need 2-4x the workgroups for the same bytes (4-byte
    // vectors: 96 against 107 us with one).
    bool four = kernel == GGRMS_KERNEL_WAVE && vb < 16;
    if (flags & GGRMS_FLAG_WAVE_ONE) four = false;
    if (kernel == GGRMS_KERNEL_WAVE && (flags & GGRMS_FLAG_WAVE_FOUR)) four = true;
    int block = four ? kWaveBlock : kWaveBlockOneWave;
    plan->pub.block_threads = block;
    // Tile order: XCD-banded when each group has its own weights and the
    // row-major order would not keep every XCD on a fixed set of columns --
    // i.e. unless a row is a whole multiple of 8 workgroups (row-major WAVE
    // workgroups take a linear run of units, so rows line up with them only
    // if the groups per workgroup divide the row).
    int64_t R1, C1;
    launch_tiles(*plan, rows, &R1, &C1);
    const int64_t gpwg = kernel == GGRMS_KERNEL_WAVE ? wave_groups_per_workgroup(lanes, block) : 1;
    const int64_t tiles_per_row = kernel == GGRMS_KERNEL_RUN ? plan->runs_per_row : groups;
    const bool orderable = kernel != GGRMS_KERNEL_WIDE && kernel != GGRMS_KERNEL_ROWS;
    plan->xband = orderable && !(flags & GGRMS_FLAG_WEIGHT_PER_GROUP) &&
                  tiles_per_row % (kXcds * gpwg) != 0;
    // Packed groups in one-wave WAVE workgroups or in runs: a tile's bytes
    // (its groups' bytes) are not a multiple of the 128-byte cache line, so
    // neighbouring tiles of a row share a line at their edge.  Run by different XCDs, both
    // L2s fetch that line and each writes back its part (377 MB of 100-wide
    // fp16 groups in 800-byte tiles: 8% more bytes fetched than the inputs
    // hold, 116K partial-line writes).  The banded order then deals S
    // consecutive tiles of a row to one XCD together -- S the smallest power
    // of two with S tiles a whole number of lines, or the largest power of
    // two below it that divides the row's tiles -- and is taken for such jobs
    // whatever the row's tile count.  Runs of 8 127-wide bf16 groups (2032
    // bytes, 6 runs per row: super-tiles of 2): fetched bytes 1.072 -> 1.050x
    // the inputs', same time (70.6 / 70.8 us).
    int64_t super = 1;
    if (((kernel == GGRMS_KERNEL_WAVE && block == kWaveBlockOneWave) ||
         kernel == GGRMS_KERNEL_RUN) &&
        packed && !(flags & GGRMS_FLAG_ORDER_ROWS)) {
        const int64_t tile_bytes = (kernel == GGRMS_KERNEL_RUN ? gpw : gpwg) * gbytes;
        while ((super * tile_bytes) % 128 != 0) super <<= 1;
        while (super > 1 && C1 % super != 0) super >>= 1;
        if (super > 1) plan->xband = true;
    }
    if (flags & GGRMS_FLAG_ORDER_ROWS) plan->xband = false;
    if ((flags & GGRMS_FLAG_ORDER_BANDED) && orderable) plan->xband = true;
    plan->super_shift = 0;
    if (plan->xband)
        while ((int64_t)1 << plan->super_shift < super) ++plan->super_shift;
    if (kernel == GGRMS_KERNEL_BLOCK) block = lanes * upb;
    if (kernel == GGRMS_KERNEL_WIDE) block = kWideBlock;
    if (kernel == GGRMS_KERNEL_RUN) block = 64;
    if (kernel == GGRMS_KERNEL_ROWS) block = lanes;
    plan->pub.block_threads = block;
    // ROWS: S workgroups per group, S <= rows; workgroup b takes rows
    // b / groups + k * S of group b % groups.
    if (kernel == GGRMS_KERNEL_ROWS) {
        int64_t S = kRowsWorkgroups / groups;
        if (S < 1) S = 1;
        if (S > rows) S = rows;
        plan->rows_stride = S;
    }
    // Threads per row of the grid.  Each launch stays within 2^31 threads
    // (so within 2^31 units and tiles too) and the kernels index with 32-bit
    // integers; larger jobs are split by rows.
    int64_t row_threads = groups * (kernel == GGRMS_KERNEL_WIDE ? kWideBlock : lanes);
    if (kernel == GGRMS_KERNEL_RUN) row_threads = plan->runs_per_row * 64;
    if (kernel == GGRMS_KERNEL_WAVE && plan->xband) row_threads = C1 * block;
    int64_t rows_per_launch = ((int64_t)1 << 31) / row_threads;
    if (rows_per_launch < 1) return GGRMS_ERROR_INVALID_VALUE;  // one row alone too large
    if (rows_per_launch > rows || kernel == GGRMS_KERNEL_ROWS) rows_per_launch = rows;
    const int64_t launches = (rows + rows_per_launch - 1) / rows_per_launch;
    int64_t workgroups = 0;
    for (int64_t r0 = 0; r0 < rows; r0 += rows_per_launch) {
        const int64_t r = rows - r0 < rows_per_launch ? rows - r0 : rows_per_launch;
        workgroups += launch_workgroups(*plan, r);
    }
    plan->nvec = nvec;
    plan->rows_per_launch = rows_per_launch;
    plan->pub.kernel = kernel;
    plan->pub.vector_bytes = vb;
    plan->pub.piece_bytes = pb;
    plan->pub.lanes_per_group = lanes;
    plan->pub.vectors_per_lane = vpt;
    plan->pub.block_threads = block;
    plan->pub.launches = (int32_t)launches;
    plan->pub.rows_per_workgroup = upb;
    if (kernel == GGRMS_KERNEL_ROWS)
        plan->pub.rows_per_workgroup = (int32_t)((rows + plan->rows_stride - 1) / plan->rows_stride);
    plan->pub.lds_bytes = upb > 1 ? (int32_t)(group_size * 4) : 0;
    if (kernel == GGRMS_KERNEL_RUN && (flags & GGRMS_FLAG_WEIGHT_PER_GROUP))
        plan->pub.lds_bytes = (int32_t)(group_size * 4);  // the staged shared weight
    plan->pub.workgroups = workgroups;
    plan->pub.tile_order = plan->xband ? 1 : 0;
    plan->pub.super_tile = 1 << plan->super_shift;
    // Cache policy: stream large jobs, keep small ones cached.  The job is
    // 3 * rows * row_bytes bytes; rows * row_bytes is at most y's extent, so
    // it does not overflow, and comparing it with ceil(min / 3) is exact.
    if (flags & GGRMS_FLAG_CACHE_STREAM)
        plan->pub.streaming = 1;
    else if (flags & GGRMS_FLAG_CACHE_KEEP)
        plan->pub.streaming = 0;
    else
        plan->pub.streaming = rows * row_bytes >= (GGRMS_STREAM_MIN_BYTES + 2) / 3 ? 1 : 0;
    return GGRMS_SUCCESS;
}

}  // namespace ggrms

extern "C" ggrms_status_t ggrms_plan_tuned(const void* y, const void* gate,
                                           const float* norm_weight, void* out, int64_t rows,
                                           int64_t width, int64_t group_size,
                                           int64_t y_row_stride, int64_t gate_row_stride,
                                           int64_t out_row_stride, float eps, ggrms_dtype_t dtype,
                                           uint32_t flags, const ggrms_shape_t* shape,
                                           ggrms_plan_t* plan) {
    if (!plan) return GGRMS_ERROR_INVALID_VALUE;
    ggrms::LaunchPlan lp;
    const ggrms_status_t st = ggrms::make_plan(y, gate, norm_weight, out, rows, width, group_size,
                                               y_row_stride, gate_row_stride, out_row_stride, eps,
                                               (int)dtype, flags, shape, &lp);
    if (st == GGRMS_SUCCESS) *plan = lp.pub;
    return st;
}

extern "C" ggrms_status_t ggrms_plan_ex(const void* y, const void* gate,
                                        const float* norm_weight, void* out, int64_t rows,
                                        int64_t width, int64_t group_size, int64_t y_row_stride,
                                        int64_t gate_row_stride, int64_t out_row_stride,
                                        float eps, ggrms_dtype_t dtype, uint32_t flags,
                                        ggrms_plan_t* plan) {
    if (flags & ~ggrms::kOperatorFlags) return GGRMS_ERROR_INVALID_VALUE;
    return ggrms_plan_tuned(y, gate, norm_weight, out, rows, width, group_size, y_row_stride,
                            gate_row_stride, out_row_stride, eps, dtype, flags, nullptr, plan);
}

extern "C" ggrms_status_t ggrms_plan(const void* y, const void* gate, const float* norm_weight,
                                     void* out, int64_t rows, int64_t width, int64_t group_size,
                                     int64_t y_row_stride, int64_t gate_row_stride,
                                     int64_t out_row_stride, float eps, ggrms_dtype_t dtype,
                                     int round_intermediate, ggrms_plan_t* plan) {
    if (round_intermediate != 0 && round_intermediate != 1) return GGRMS_ERROR_INVALID_VALUE;
    return ggrms_plan_tuned(y, gate, norm_weight, out, rows, width, group_size, y_row_stride,
                            gate_row_stride, out_row_stride, eps, dtype,
                            round_intermediate ? GGRMS_FLAG_ROUND_INTERMEDIATE : 0u, nullptr, plan);
}

extern "C" const char* ggrms_status_string(ggrms_status_t status) {
    switch (status) {
    case GGRMS_SUCCESS: return "success";
    case GGRMS_ERROR_INVALID_VALUE: return "invalid argument";
    case GGRMS_ERROR_NOT_SUPPORTED: return "not supported (dtype or device)";
    case GGRMS_ERROR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

extern "C" int ggrms_abi_version(void) { return GGRMS_ABI_VERSION; }
