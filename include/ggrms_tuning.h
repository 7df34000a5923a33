/*
 * ggrms_tuning.h -- launch controls of libggrms.so, for tuning sweeps,
 * measurements and cross-checks of the kernel families against each other.
 *
 * Nothing here changes what is computed: whatever these controls select, the
 * outputs meet the accuracy stated in ggrms.h, and launches that differ only
 * in cache policy, tile order or WAVE workgroup size give identical bits.
 * Applications call ggrms_forward / ggrms_forward_ex (ggrms.h), which choose
 * all of this themselves.
 */
#ifndef GGRMS_TUNING_H
#define GGRMS_TUNING_H

#include "ggrms.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Flags beyond ggrms_flag_t, taken by the _tuned calls only (the _ex calls
 * reject them).  Setting both flags of one pair is GGRMS_ERROR_INVALID_VALUE. */
typedef enum {
    /* Cache policy for y, gate and out: CACHE_STREAM forces the
     * non-temporal hint, CACHE_KEEP forces plain accesses, overriding the
     * default by job size (GGRMS_STREAM_MIN_BYTES, ggrms.h). */
    GGRMS_FLAG_CACHE_STREAM = 8,
    GGRMS_FLAG_CACHE_KEEP = 16,
    /* Tile order (plan field tile_order): ORDER_ROWS / ORDER_BANDED force
     * the row-major or the XCD-banded order (no effect on WIDE and ROWS,
     * whose workgroups take their own rows). */
    GGRMS_FLAG_ORDER_ROWS = 32,
    GGRMS_FLAG_ORDER_BANDED = 64,
    /* WAVE workgroups of one or four waves (by default one for 16-byte
     * vectors, packed groups included, and four for narrower vectors; no
     * effect on BLOCK, WIDE, RUN and ROWS). */
    GGRMS_FLAG_WAVE_ONE = 128,
    GGRMS_FLAG_WAVE_FOUR = 256
} ggrms_tuning_flag_t;

/*
 * A kernel shape.  All zero: the library chooses everything.  Otherwise:
 *
 *   lanes_per_group   1, 2, 4, ..., 64 (WAVE kernel) or 128, 256, 512, 1024
 *                     (BLOCK kernel; 1024 with vectors_per_lane = 0 is WIDE);
 *                     0 together with vectors_per_lane = 0: the library
 *                     chooses lanes and vectors for the vector width below
 *   vectors_per_lane  1 for lanes < 64; 1..4 for 64 lanes or the BLOCK
 *                     kernel (also 6 with 256 lanes); 0 for WIDE
 *   rows_per_workgroup  0 to let the library choose; 1; or, for the BLOCK
 *                     kernel, 2 or 4 with 128 lanes and 2 with 256 lanes (the
 *                     workgroup's rows share one group, whose weights are
 *                     staged once in LDS; needs a 16-byte aligned weight and
 *                     group_size % 4 == 0)
 *   vector_bytes      0 for the widest vector the alignment allows; or 16,
 *                     8, 4 or 2 (at least the element size): every y/gate/out
 *                     access is a vector of that size, which the pointers,
 *                     row strides and the group's byte length must allow
 *                     (16 also allows packed groups, see ggrms.h)
 *   kernel            0: the kernel family follows from lanes and vectors;
 *                     GGRMS_KERNEL_RUN: runs of packed groups (lanes and
 *                     vectors 0, or 64 and 1 or 2; two groups must fit in
 *                     64 x vectors slots);
 *                     GGRMS_KERNEL_ROWS: rows in turn per workgroup, for
 *                     16-byte vectors that are not packed (lanes and vectors
 *                     0 for the library's choice, or 256 x 3, 320 x 2,
 *                     384 x 2, 448 x 2, 512 x 2, 768 x 2, 1024 x 2;
 *                     rows_per_workgroup 0 or 1)
 *
 * For packed groups the shape must cover the vectors of the worst-aligned
 * group, WIDE is not built and rows_per_workgroup must be 0 or 1.
 */
typedef struct {
    int32_t lanes_per_group;
    int32_t vectors_per_lane;
    int32_t rows_per_workgroup;
    int32_t vector_bytes;
    int32_t kernel;
} ggrms_shape_t;

/*
 * ggrms_forward_tuned -- ggrms_forward_ex with launch controls: `flags` may
 * also hold ggrms_tuning_flag_t bits, and `shape` (NULL: the library
 * chooses) forces the kernel shape.  GGRMS_ERROR_INVALID_VALUE for a shape
 * field out of range (negative, a vector_bytes that is not 0, 2, 4, 8 or 16,
 * or a kernel that is not 0, GGRMS_KERNEL_RUN or GGRMS_KERNEL_ROWS);
 * GGRMS_ERROR_NOT_SUPPORTED for a shape that is not built, whose
 * lanes_per_group * vectors_per_lane vectors do not cover one group, whose
 * rows_per_workgroup cannot be used, or whose vector_bytes the alignment
 * does not allow.  Otherwise as ggrms_forward_ex.
 */
GGRMS_API ggrms_status_t ggrms_forward_tuned(const void* y, const void* gate,
                                             const float* norm_weight, void* out, int64_t rows,
                                             int64_t width, int64_t group_size,
                                             int64_t y_row_stride, int64_t gate_row_stride,
                                             int64_t out_row_stride, float eps,
                                             ggrms_dtype_t dtype, uint32_t flags,
                                             const ggrms_shape_t* shape, void* stream);

/* ggrms_plan for ggrms_forward_tuned's arguments (no HIP call). */
GGRMS_API ggrms_status_t ggrms_plan_tuned(const void* y, const void* gate,
                                          const float* norm_weight, void* out, int64_t rows,
                                          int64_t width, int64_t group_size, int64_t y_row_stride,
                                          int64_t gate_row_stride, int64_t out_row_stride,
                                          float eps, ggrms_dtype_t dtype, uint32_t flags,
                                          const ggrms_shape_t* shape, ggrms_plan_t* plan);

#ifdef __cplusplus
}
#endif

#endif /* GGRMS_TUNING_H */
