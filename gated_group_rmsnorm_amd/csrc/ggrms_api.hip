// ggrms_api.hip -- ggrms_forward: checks, device check, kernel launches.
//
// The host side is deliberately thin: make_plan (plan.cpp) validates and
// picks the kernel shape without touching the device; this file confirms the
// current device is gfx950 (cached per device), fills the kernel arguments
// and enqueues one launch per row chunk on the caller's stream.  No
// allocation, no synchronisation, nothing that would break stream capture
// after the first call on a device.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "ggrms.h"
#include "ggrms_internal.h"
#include "ggrms_tuning.h"

namespace ggrms {
namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

bool device_is_gfx950() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
    int st = dev < kMaxDevices ? g_device_state[dev].load(std::memory_order_acquire) : 0;
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
        st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        if (dev < kMaxDevices) g_device_state[dev].store(st, std::memory_order_release);
    }
    return st == 1;
}

const void* pick(int dtype, bool nbg, bool nt, int kernel, int vb, int pb, int lanes, int vpt,
                 int upb) {
    switch (dtype) {
    case GGRMS_F32: return (nbg ? pick_f32_nbg : pick_f32)(kernel, vb, pb, lanes, vpt, upb, nt);
    case GGRMS_F16: return (nbg ? pick_f16_nbg : pick_f16)(kernel, vb, pb, lanes, vpt, upb, nt);
    case GGRMS_BF16: return (nbg ? pick_bf16_nbg : pick_bf16)(kernel, vb, pb, lanes, vpt, upb, nt);
    default: return nullptr;
    }
}

ggrms_status_t forward_impl(const void* y, const void* gate, const float* norm_weight, void* out,
                            int64_t rows, int64_t width, int64_t group_size, int64_t y_row_stride,
                            int64_t gate_row_stride, int64_t out_row_stride, float eps,
                            ggrms_dtype_t dtype, uint32_t flags, const ggrms_shape_t* shape,
                            void* stream) {
    LaunchPlan lp;
    ggrms_status_t st = make_plan(y, gate, norm_weight, out, rows, width, group_size, y_row_stride,
                                  gate_row_stride, out_row_stride, eps, (int)dtype, flags, shape,
                                  &lp);
    if (st != GGRMS_SUCCESS || lp.pub.kernel == GGRMS_KERNEL_NONE) return st;
    if (!device_is_gfx950()) return GGRMS_ERROR_NOT_SUPPORTED;

    const ggrms_plan_t& p = lp.pub;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool nbg = (flags & GGRMS_FLAG_NORM_BEFORE_GATE) != 0;
    // (ROWS reports the rows each workgroup takes in turn; its kernels are
    // built for one unit at a time)
    const void* fn = pick((int)dtype, nbg, p.streaming != 0, p.kernel, p.vector_bytes,
                          p.piece_bytes, p.lanes_per_group, p.vectors_per_lane,
                          p.kernel == GGRMS_KERNEL_ROWS ? 1 : p.rows_per_workgroup);
    if (!fn) return GGRMS_ERROR_NOT_SUPPORTED;

    if (rows == 1) y_row_stride = gate_row_stride = out_row_stride = width;
    KArgs a;
    a.w = norm_weight;
    a.sy = y_row_stride;
    a.sg = gate_row_stride;
    a.so = out_row_stride;
    a.groups = (uint32_t)lp.groups;
    uint32_t div_s = 0, xc_s = 0;
    // the row of a row-major tile: x / groups, or (RUN) x / runs per row
    div_magic(p.kernel == GGRMS_KERNEL_RUN ? (uint32_t)lp.runs_per_row : a.groups, &a.div_m, &div_s);
    a.G = (uint32_t)group_size;
    a.nvec = (uint32_t)lp.nvec;
    a.Ginv = (float)(1.0 / (double)group_size);
    a.eps = eps;
    // tile columns of the banded order (the same for every launch of the job)
    int64_t R, C;
    launch_tiles(lp, lp.rows_per_launch, &R, &C);
    (void)R;
    // (ROWS: the step between a workgroup's rows)
    a.xc = p.kernel == GGRMS_KERNEL_ROWS ? (uint32_t)lp.rows_stride : (uint32_t)C;
    div_magic(a.xc, &a.xc_m, &xc_s);
    a.bits = (div_s << kBitDivShift) | (xc_s << kBitXcShift) |
             ((dtype != GGRMS_F32 && (flags & GGRMS_FLAG_ROUND_INTERMEDIATE)) ? kBitRound : 0u) |
             ((flags & GGRMS_FLAG_WEIGHT_PER_GROUP) ? kBitShared : 0u) | (lp.xband ? kBitBand : 0u) |
             ((uint32_t)lp.super_shift << kBitSuperShift);
    const int es = lp.esize;

    for (int64_t r0 = 0; r0 < rows; r0 += lp.rows_per_launch) {
        const int64_t r = rows - r0 < lp.rows_per_launch ? rows - r0 : lp.rows_per_launch;
        a.y = static_cast<const char*>(y) + r0 * y_row_stride * es;
        a.gate = static_cast<const char*>(gate) + r0 * gate_row_stride * es;
        a.out = static_cast<char*>(out) + r0 * out_row_stride * es;
        a.rows = (uint32_t)r;
        const int64_t blocks = launch_workgroups(lp, r);
        void* args[] = {&a};
        if (hipLaunchKernel(fn, dim3((uint32_t)blocks), dim3((uint32_t)p.block_threads), args,
                            (size_t)p.lds_bytes, s) != hipSuccess)
            return GGRMS_ERROR_LAUNCH;
    }
    return GGRMS_SUCCESS;
}

}  // namespace
}  // namespace ggrms

extern "C" ggrms_status_t ggrms_forward_tuned(const void* y, const void* gate,
                                              const float* norm_weight, void* out, int64_t rows,
                                              int64_t width, int64_t group_size,
                                              int64_t y_row_stride, int64_t gate_row_stride,
                                              int64_t out_row_stride, float eps,
                                              ggrms_dtype_t dtype, uint32_t flags,
                                              const ggrms_shape_t* shape, void* stream) {
    return ggrms::forward_impl(y, gate, norm_weight, out, rows, width, group_size, y_row_stride,
                               gate_row_stride, out_row_stride, eps, dtype, flags, shape, stream);
}

extern "C" ggrms_status_t ggrms_forward_ex(const void* y, const void* gate,
                                           const float* norm_weight, void* out, int64_t rows,
                                           int64_t width, int64_t group_size,
                                           int64_t y_row_stride, int64_t gate_row_stride,
                                           int64_t out_row_stride, float eps, ggrms_dtype_t dtype,
                                           uint32_t flags, void* stream) {
    if (flags & ~ggrms::kOperatorFlags) return GGRMS_ERROR_INVALID_VALUE;
    return ggrms::forward_impl(y, gate, norm_weight, out, rows, width, group_size, y_row_stride,
                               gate_row_stride, out_row_stride, eps, dtype, flags, nullptr,
                               stream);
}

extern "C" ggrms_status_t ggrms_forward(const void* y, const void* gate,
                                        const float* norm_weight, void* out, int64_t rows,
                                        int64_t width, int64_t group_size, int64_t y_row_stride,
                                        int64_t gate_row_stride, int64_t out_row_stride,
                                        float eps, ggrms_dtype_t dtype, int round_intermediate,
                                        void* stream) {
    if (round_intermediate != 0 && round_intermediate != 1) return GGRMS_ERROR_INVALID_VALUE;
    return ggrms::forward_impl(y, gate, norm_weight, out, rows, width, group_size, y_row_stride,
                               gate_row_stride, out_row_stride, eps, dtype,
                               round_intermediate ? GGRMS_FLAG_ROUND_INTERMEDIATE : 0u, nullptr,
                               stream);
}
