/*
 * ggrms.h -- C ABI of the fused gated group-RMSNorm library (libggrms.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation.  The page "gated_group_rmsnorm" (Mojo module doc on
 * max.modular.com; the math block after its intro and the paragraph after
 * it) defines, for a row n of the intermediate axis split into contiguous
 * groups of group_size = G columns, group g, col = g*G + j:
 *
 *     gated = f32(y[n,col]) * silu(f32(gate[n,col]))      f32
 *     m2    = sum over the G columns of gated^2           f32
 *     nf    = rsqrt(m2 / G + eps)                        eps added after the mean
 *     out[n,col] = cast(f32(norm_weight[col]) * f32(cast(gated*nf, y.dtype)), out.dtype)
 *
 * This computes the Mamba-2 mixer's gated RMSNorm in its norm_before_gate =
 * False form; one launch replaces the four-op chain (widen, silu-gate, group
 * RMSNorm, weight multiply and narrow) the page's intro describes.  With
 * round_intermediate = 0 the intermediate cast(gated*nf, y.dtype) is skipped
 * and every intermediate stays f32 until the final store (the mode that the
 * page "com.microsoft.GatedRMSNorm", Description section, describes for its
 * operator).  Casts round to nearest, ties to even, keep subnormals and
 * overflow to infinity.  Accuracy: against the formula evaluated step by step
 * in f32 with correctly rounded operations, f32 outputs agree within a
 * relative 1e-5 and bf16/fp16 outputs within 2 units in the last place (the
 * group sum's order, silu's exp and reciprocal and the normaliser's rsqrt
 * each differ by a few f32 ulp; two narrowing casts can each fall on the
 * other side of a tie).  Results are deterministic run to run.
 *
 * Layout.  y, gate and out are row-major [rows, width] views with unit column
 * stride and their own row strides, so y and gate may be column slices of one
 * fused in-projection buffer (the page's Parallelization section reads strided
 * views directly).  Rows are tokens of one or more sequences of any lengths,
 * flattened into one axis (the page's intro: the op stands alone and takes
 * variable-length batches); leading axes fold into rows.
 *
 * Threading and ownership.  The caller owns every buffer.  The library
 * allocates nothing, frees nothing, keeps no pointer after a call returns,
 * never synchronises, and is safe to call from several threads at once.
 * ggrms_forward only enqueues work on `stream` and returns (as the page's
 * Functions section describes its GPU entry point); results are ready when
 * the stream reaches that point.  Faults inside the kernel surface at the caller's next
 * synchronisation with that stream.  A call may be captured into a HIP graph
 * (stream capture) and replayed: it allocates nothing, waits for nothing and
 * enqueues nothing but its kernel launches, whose arguments are fixed at
 * capture.  The current device's architecture is queried on the first call
 * on that device and cached.
 */
#ifndef GGRMS_H
#define GGRMS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GGRMS_ABI_VERSION 5

/* The library exports the functions declared here and in ggrms_tuning.h
 * (launch controls for tuning and cross-checks) and nothing else (it is
 * built with hidden visibility). */
#if defined(__GNUC__)
#define GGRMS_API __attribute__((visibility("default")))
#else
#define GGRMS_API
#endif

/* Element type shared by y, gate and out.  The weight is always f32. */
typedef enum {
    GGRMS_F32 = 0,  /* IEEE binary32 */
    GGRMS_F16 = 1,  /* IEEE binary16 */
    GGRMS_BF16 = 2  /* bfloat16: the upper 16 bits of a binary32 */
} ggrms_dtype_t;

typedef enum {
    GGRMS_SUCCESS = 0,
    /* An argument violates the contract below; nothing was enqueued. */
    GGRMS_ERROR_INVALID_VALUE = 1,
    /* Unknown dtype, or the current device is not gfx950; nothing was enqueued. */
    GGRMS_ERROR_NOT_SUPPORTED = 2,
    /* The HIP runtime refused a kernel launch. */
    GGRMS_ERROR_LAUNCH = 3
} ggrms_status_t;

/*
 * ggrms_forward -- enqueue the fused gated group-RMSNorm on `stream`.
 *
 *   y, gate       device pointers to the first element of [rows, width]
 *                 views of `dtype`; read only.  They may overlap each other.
 *   norm_weight   device pointer to `width` f32 values, indexed by column;
 *                 read only; 4-byte aligned.
 *   out           device pointer to the first element of a [rows, width]
 *                 view of `dtype`; every element of the view is written,
 *                 nothing outside it is touched.  out may be exactly y or
 *                 exactly gate (same pointer and same row stride: in place);
 *                 any other overlap with y or gate, and any overlap with
 *                 norm_weight (which every row reads), is rejected.
 *   rows          number of rows (tokens), >= 0.  rows == 0 enqueues nothing.
 *   width         columns per row, > 0, a multiple of group_size.
 *   group_size    columns per normalisation group (G), > 0.
 *   *_row_stride  distance between consecutive rows, in elements; >= width
 *                 when rows > 1 (ignored when rows == 1).
 *   eps           added to the mean of squares; finite and >= 0.
 *   dtype         a ggrms_dtype_t.
 *   round_intermediate
 *                 1: cast gated*nf to `dtype` and back before the weight
 *                 multiply; 0: keep it f32.  For GGRMS_F32 both are identical.
 *   stream        a hipStream_t, or NULL for the null stream.
 *
 * The buffers and the stream belong to the calling thread's current HIP
 * device, which is the device that is checked and launched on.  Every
 * element pointer must be aligned to its element size.
 *
 * Returns GGRMS_SUCCESS once the work is enqueued.  Argument checks run
 * before any HIP call: GGRMS_ERROR_INVALID_VALUE for a negative rows, a
 * non-positive width or group_size, width % group_size != 0, a NULL pointer
 * when rows > 0, a row stride < width when rows > 1, a misaligned pointer,
 * round_intermediate other than 0 or 1, a NaN, infinite or negative eps,
 * extents that overflow 64-bit addressing, or a disallowed overlap of out
 * with y, gate or norm_weight; GGRMS_ERROR_NOT_SUPPORTED for an unknown
 * dtype.  Then the current device is checked (GGRMS_ERROR_NOT_SUPPORTED
 * unless gfx950) and the kernels are launched (GGRMS_ERROR_LAUNCH if the
 * runtime refuses one).
 */
GGRMS_API ggrms_status_t ggrms_forward(const void* y, const void* gate, const float* norm_weight,
                                       void* out, int64_t rows, int64_t width, int64_t group_size,
                                       int64_t y_row_stride, int64_t gate_row_stride,
                                       int64_t out_row_stride, float eps, ggrms_dtype_t dtype,
                                       int round_intermediate, void* stream);

/* Which kernel ggrms_forward would launch for a set of arguments. */
typedef enum {
    GGRMS_KERNEL_NONE = 0,   /* rows == 0: nothing to launch */
    GGRMS_KERNEL_WAVE = 1,   /* one span of <= 64 lanes per (row, group); no LDS, no barrier */
    GGRMS_KERNEL_BLOCK = 2,  /* one (row, group) across 2..16 waves; LDS combine, one barrier */
    GGRMS_KERNEL_WIDE = 3,   /* groups too wide for registers: two passes over the group */
    GGRMS_KERNEL_RUN = 4,    /* packed groups: one wave over a run of consecutive groups of a
                                row, one or two vectors per lane; group sums in LDS */
    GGRMS_KERNEL_ROWS = 5    /* wide groups in large jobs: one workgroup per compute unit
                                takes rows of one group in turn, the next rows' inputs in
                                flight while it stores; LDS combine, one barrier per row */
} ggrms_kernel_t;

typedef struct {
    int32_t kernel;           /* a ggrms_kernel_t */
    int32_t vector_bytes;     /* bytes per y/gate/out load (16, 8, 4 or 2) */
    int32_t lanes_per_group;  /* lanes that share one (row, group) */
    int32_t vectors_per_lane; /* vectors each lane holds per group (0 for WIDE: it loops) */
    int32_t block_threads;    /* threads per workgroup */
    int32_t launches;         /* kernel launches (rows are split if a grid would be too large) */
    int32_t rows_per_workgroup; /* BLOCK: rows of one group per workgroup (weights shared in
                                   LDS); ROWS: the most rows one workgroup takes in turn */
    int32_t lds_bytes;        /* dynamic LDS per workgroup (the staged weights) */
    int64_t workgroups;       /* workgroups over all launches */
    int32_t streaming;        /* 1: y/gate/out loads and stores carry the non-temporal hint
                                 (the default for jobs of at least GGRMS_STREAM_MIN_BYTES) */
    int32_t piece_bytes;      /* == vector_bytes when every group starts on a vector
                                 boundary; 2, 4 or 8 for packed groups (see below) */
    int32_t tile_order;       /* order in which workgroups take the job's tiles:
                                 0 row-major, 1 XCD-banded (see below) */
    int32_t groups_per_run;   /* RUN: groups one wave takes (the last run of a row may
                                 hold fewer); 0 for the other kernels */
    int32_t super_tile;       /* XCD-banded order: consecutive tiles of a row dealt to one
                                 XCD together, so that tiles sharing cache lines meet in
                                 one L2 (> 1 only for packed groups in one-wave WAVE
                                 workgroups or in runs); 1 otherwise */
} ggrms_plan_t;

/*
 * Vector width.  Every y/gate/out access is a vector of the widest size
 * (16, 8, 4 or 2 bytes) that the three base pointers, their row strides, the
 * group's byte length and the weight's alignment allow.  When the group's
 * byte length is not a multiple of 16 (say 100 fp16 values, 200 bytes) but
 * more than 16, and the rows are: every base pointer and row stride 16-byte
 * aligned, width * element size a multiple of 16, and a per-column weight
 * 16-byte aligned or one weight shared by every group (read by element) --
 * the groups are "packed": 16-byte vectors are counted from
 * the start of the row, a vector on a group boundary is read by both groups
 * (each uses its own elements) and written in pieces of
 * piece_bytes = gcd(group bytes, 16), so no element is written twice and no
 * read leaves the row.  In a large job, packed groups that would leave most
 * of their lane segment idle (RUN) are taken a run of consecutive groups per
 * wave, the lanes holding the run's vectors one or two each; a run of a
 * whole number of vectors is stored in whole vectors, another one only in
 * pieces at its two ends.
 */

/*
 * Tile order.  Row-major: workgroup b takes the b-th tile (WAVE: the next
 * units of the (row, group) sequence; BLOCK: row tile b / groups, group
 * b % groups).  XCD-banded, chosen when every group has its own weights and
 * a row does not split into a multiple of 8 full tiles (WIDE launches are
 * always row-major): the tiles are taken in blocks of 8
 * rows, and the part's 8 XCDs (workgroup b runs on XCD b % 8) each take a
 * band of about 1/8 of the columns of every block, so each XCD reads the
 * weights of its band only, while the tiles in flight still cover a
 * contiguous run of rows.  Results are identical in either order.
 */

/*
 * ggrms_plan -- run ggrms_forward's argument checks and kernel choice
 * without touching the device; fills *plan on GGRMS_SUCCESS.  Makes no HIP
 * call, so it works on a host without a GPU.
 */
GGRMS_API ggrms_status_t ggrms_plan(const void* y, const void* gate, const float* norm_weight,
                                    void* out, int64_t rows, int64_t width, int64_t group_size,
                                    int64_t y_row_stride, int64_t gate_row_stride,
                                    int64_t out_row_stride, float eps, ggrms_dtype_t dtype,
                                    int round_intermediate, ggrms_plan_t* plan);

/* Operator variants (bits of the `flags` argument of the _ex calls). */
typedef enum {
    /* Gate first (the default): cast gated*nf to dtype and back before the
     * weight multiply.  Same as round_intermediate = 1. */
    GGRMS_FLAG_ROUND_INTERMEDIATE = 1,
    /* Norm first: out = cast(((y * nf) * w) * silu(gate)) with
     * nf = rsqrt(sum y^2 / G + eps) and every intermediate f32 -- the
     * operator of the page "com.microsoft.GatedRMSNorm" (Description
     * section).  Not combinable with GGRMS_FLAG_ROUND_INTERMEDIATE. */
    GGRMS_FLAG_NORM_BEFORE_GATE = 2,
    /* norm_weight holds group_size values shared by every group (indexed by
     * the column within the group), as that page's `scale` input does;
     * without it, width values indexed by the column. */
    GGRMS_FLAG_WEIGHT_PER_GROUP = 4
} ggrms_flag_t;

/* Cache policy.  y, gate and out are each touched once per call.  A job
 * whose y, gate and out views hold at least GGRMS_STREAM_MIN_BYTES together
 * is streamed: its loads and stores carry the non-temporal hint, which keeps
 * a large one-pass stream from evicting other data and runs it faster.
 * Smaller jobs (decode) use plain accesses, so inputs still cached from the
 * kernel that wrote them are hit and the output stays cached for the kernel
 * that reads it next.  The weight is always cached.  Results do not depend
 * on the policy. */
#define GGRMS_STREAM_MIN_BYTES (4ll << 20)

/*
 * ggrms_forward_ex -- ggrms_forward with operator flags (a mask of
 * ggrms_flag_t) instead of round_intermediate.  The weight needs width
 * values, or group_size with GGRMS_FLAG_WEIGHT_PER_GROUP.
 * GGRMS_ERROR_INVALID_VALUE also for unknown flag bits (including the launch
 * controls of ggrms_tuning.h, which only ggrms_forward_tuned takes) and for
 * GGRMS_FLAG_ROUND_INTERMEDIATE with GGRMS_FLAG_NORM_BEFORE_GATE.
 */
GGRMS_API ggrms_status_t ggrms_forward_ex(const void* y, const void* gate, const float* norm_weight,
                                          void* out, int64_t rows, int64_t width,
                                          int64_t group_size, int64_t y_row_stride,
                                          int64_t gate_row_stride, int64_t out_row_stride,
                                          float eps, ggrms_dtype_t dtype, uint32_t flags,
                                          void* stream);

/* ggrms_plan for ggrms_forward_ex's arguments (no HIP call). */
GGRMS_API ggrms_status_t ggrms_plan_ex(const void* y, const void* gate, const float* norm_weight,
                                       void* out, int64_t rows, int64_t width, int64_t group_size,
                                       int64_t y_row_stride, int64_t gate_row_stride,
                                       int64_t out_row_stride, float eps, ggrms_dtype_t dtype,
                                       uint32_t flags, ggrms_plan_t* plan);

/* Static, NUL-terminated description of a status code (never NULL). */
GGRMS_API const char* ggrms_status_string(ggrms_status_t status);

/* GGRMS_ABI_VERSION of the loaded library. */
GGRMS_API int ggrms_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GGRMS_H */
