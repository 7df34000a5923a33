// bench_aux.hip -- measurement helpers for the benchmark (libggrms_bench.so).
// Not part of the product ABI.
//   * an empty kernel taking an argument block of the same size as the
//     normalisation kernels, launched with a caller-chosen grid: the floor
//     that a decode launch is compared against;
//   * decode bursts issued from C through libggrms.so's ggrms_forward_tuned
//     (eager and replayed as one HIP graph; the library's own launch
//     choice unless the caller forces a shape), next to the same bursts of the
//     empty kernel, so the per-launch figure carries no interpreter overhead;
//   * a plain 16-byte vector copy of known size: the calibration that turns
//     the FETCH_SIZE / WRITE_SIZE counters into HBM bytes;
//   * whole jobs (the fused kernel or the plain stream kernel) launched back
//     to back from C, for jobs small enough that a launch from the
//     interpreter takes longer than the kernel;
//   * the simplest kernel that moves a workload's bytes: two streams read and
//     one written, 16-byte non-temporal accesses, one vector per lane,
//     one-wave workgroups (the fastest plain form in a sweep of vectors per
//     lane 1-4, workgroups of 64-1024 threads and cache hints: 0.82-0.83 of
//     HBM peak at 377 MB, against 0.80-0.81 with 2 vectors per lane in
//     256-thread workgroups) -- the practical ceiling the fused kernel is
//     compared against.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <chrono>
#include <vector>

#include "ggrms.h"
#include "ggrms_internal.h"
#include "ggrms_tuning.h"

namespace {

__global__ void ggrms_bench_empty_kernel(ggrms::KArgs) {}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void ggrms_bench_copy_kernel(const u32x4* __restrict__ src,
                                                               u32x4* __restrict__ dst,
                                                               uint64_t n) {
    const uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
    if (i < n) dst[i] = src[i];
}

// c = a ^ b over n 16-byte vectors; a one-wave workgroup takes 64
// consecutive vectors, one per lane.
__global__ __launch_bounds__(64) void ggrms_bench_stream3_kernel(const u32x4* __restrict__ a,
                                                                 const u32x4* __restrict__ b,
                                                                 u32x4* __restrict__ c,
                                                                 uint64_t n) {
    const uint64_t i = (uint64_t)blockIdx.x * 64u + threadIdx.x;
    if (i < n) {
        const u32x4 x = __builtin_nontemporal_load(a + i);
        const u32x4 y = __builtin_nontemporal_load(b + i);
        __builtin_nontemporal_store(x ^ y, c + i);
    }
}

// The same over rows x vpr 16-byte vectors of three strided views (row
// strides in 16-byte units): flat vector i is row i / vpr (a round-up
// magic-number division, m and sh from the host) and vector i % vpr of it.
// For views that are column slices of one wider buffer this reads exactly
// the bytes a fused launch over them reads, where the flat form would read
// two overlapping stretches of the buffer.
__global__ __launch_bounds__(64) void ggrms_bench_stream3_rows_kernel(
    const u32x4* __restrict__ a, const u32x4* __restrict__ b, u32x4* __restrict__ c, uint32_t n,
    uint32_t vpr, uint32_t m, uint32_t sh, uint64_t sa, uint64_t sb, uint64_t sc) {
    const uint32_t i = blockIdx.x * 64u + threadIdx.x;
    if (i < n) {
        const uint32_t r = (__umulhi(i, m) + i) >> sh;
        const uint32_t v = i - r * vpr;
        const u32x4 x = __builtin_nontemporal_load(a + r * sa + v);
        const u32x4 y = __builtin_nontemporal_load(b + r * sb + v);
        __builtin_nontemporal_store(x ^ y, c + r * sc + v);
    }
}

}  // namespace

extern "C" int ggrms_bench_empty(int64_t blocks, int threads, void* stream) {
    ggrms::KArgs a = {};
    void* args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void*>(&ggrms_bench_empty_kernel),
                           dim3((uint32_t)blocks), dim3((uint32_t)threads), args, 0,
                           static_cast<hipStream_t>(stream)) == hipSuccess
               ? 0
               : 1;
}

// Copies nbytes (a multiple of 16; both pointers 16-byte aligned).
extern "C" int ggrms_bench_copy(const void* src, void* dst, int64_t nbytes, void* stream) {
    if (nbytes <= 0 || nbytes % 16 || (uintptr_t)src % 16 || (uintptr_t)dst % 16) return 1;
    const uint64_t n = (uint64_t)nbytes / 16;
    const uint64_t blocks = (n + 255) / 256;
    if (blocks > 0xFFFFFFFFull / 256) return 1;
    void* args[] = {&src, &dst, (void*)&n};
    const u32x4* s = static_cast<const u32x4*>(src);
    u32x4* d = static_cast<u32x4*>(dst);
    args[0] = &s;
    args[1] = &d;
    return hipLaunchKernel(reinterpret_cast<const void*>(&ggrms_bench_copy_kernel),
                           dim3((uint32_t)blocks), dim3(256), args, 0,
                           static_cast<hipStream_t>(stream)) == hipSuccess
               ? 0
               : 1;
}

// c = a ^ b over nbytes per buffer (a multiple of 16; 16-byte aligned
// pointers): two reads and one write of nbytes each.
extern "C" int ggrms_bench_stream3(const void* a, const void* b, void* c, int64_t nbytes,
                                   void* stream) {
    if (nbytes <= 0 || nbytes % 16 || (uintptr_t)a % 16 || (uintptr_t)b % 16 ||
        (uintptr_t)c % 16)
        return 1;
    const uint64_t n = (uint64_t)nbytes / 16;
    const uint64_t blocks = (n + 63) / 64;
    if (blocks > 0xFFFFFFFFull / 64) return 1;  // work-items must fit in 32 bits
    const u32x4* pa = static_cast<const u32x4*>(a);
    const u32x4* pb = static_cast<const u32x4*>(b);
    u32x4* pc = static_cast<u32x4*>(c);
    void* args[] = {&pa, &pb, &pc, (void*)&n};
    return hipLaunchKernel(reinterpret_cast<const void*>(&ggrms_bench_stream3_kernel),
                           dim3((uint32_t)blocks), dim3(64), args, 0,
                           static_cast<hipStream_t>(stream)) == hipSuccess
               ? 0
               : 1;
}

// c = a ^ b over [rows, row_bytes] views with row strides sa, sb, sc in bytes
// (row_bytes and the strides multiples of 16, row_bytes <= each stride when
// rows > 1; 16-byte aligned pointers; rows * row_bytes / 16 < 2^31).
extern "C" int ggrms_bench_stream3_rows(const void* a, const void* b, void* c, int64_t rows,
                                        int64_t row_bytes, int64_t sa, int64_t sb, int64_t sc,
                                        void* stream) {
    if (rows <= 0 || row_bytes <= 0 || row_bytes % 16 || sa % 16 || sb % 16 || sc % 16 ||
        (uintptr_t)a % 16 || (uintptr_t)b % 16 || (uintptr_t)c % 16)
        return 1;
    if (rows > 1 && (sa < row_bytes || sb < row_bytes || sc < row_bytes)) return 1;
    const uint64_t vpr = (uint64_t)row_bytes / 16;
    if ((uint64_t)rows * vpr >= (1ull << 31)) return 1;
    const uint32_t n = (uint32_t)(rows * vpr);
    // x / vpr = (umulhi(x, m) + x) >> l, l = ceil(log2 vpr),
    // m = floor(2^32 (2^l - vpr) / vpr) + 1: exact for x < 2^31
    uint32_t l = 0;
    while ((1ull << l) < vpr) ++l;
    const uint32_t m = (uint32_t)(((1ull << 32) * ((1ull << l) - vpr)) / vpr + 1);
    const uint32_t d = (uint32_t)vpr;
    const uint64_t va = (uint64_t)sa / 16, vb = (uint64_t)sb / 16, vc = (uint64_t)sc / 16;
    const u32x4* pa = static_cast<const u32x4*>(a);
    const u32x4* pb = static_cast<const u32x4*>(b);
    u32x4* pc = static_cast<u32x4*>(c);
    uint32_t mm = m, ll = l;
    void* args[] = {&pa, &pb, &pc, (void*)&n, (void*)&d, &mm, &ll,
                    (void*)&va, (void*)&vb, (void*)&vc};
    return hipLaunchKernel(reinterpret_cast<const void*>(&ggrms_bench_stream3_rows_kernel),
                           dim3((n + 63) / 64), dim3(64), args, 0,
                           static_cast<hipStream_t>(stream)) == hipSuccess
               ? 0
               : 1;
}

namespace {

double median_of(std::vector<double> v) {
    std::sort(v.begin(), v.end());
    return v.empty() ? 0.0 : v[v.size() / 2];
}

// The stream, events and graph of one measurement, released on every path.
struct BurstRes {
    hipStream_t s = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    ~BurstRes() {
        if (s) hipStreamSynchronize(s);
        if (exec) hipGraphExecDestroy(exec);
        if (graph) hipGraphDestroy(graph);
        if (e0) hipEventDestroy(e0);
        if (e1) hipEventDestroy(e1);
        if (s) hipStreamDestroy(s);
    }
};

}  // namespace

// Decode bursts: `layers` back-to-back launches over the layers' [1, width]
// buffers, repeated `bursts` times on a stream of its own, after about 100 ms
// of untimed bursts (the clocks settle), with `flags` and `shape` (NULL: the
// library's choice) passed to ggrms_forward_tuned.  mode 0: eager;
// 1: the same burst captured once and replayed as a HIP graph; 2 and 3: the
// empty kernel with the fused launch's grid, eager and graph.  Device time
// comes from events around each burst (median burst / layers); host time is
// the steady-clock time of enqueueing one burst (median / layers).  Modes 4
// and 5 (fused, empty): the graph replayed `bursts` times back to back between
// two events, so that each replay's start overlaps the previous one's tail
// as in a decode loop that does not wait for every token (median of 7 such
// runs / (bursts * layers); host time 0).
// Returns 0, or a ggrms status / -1 for a HIP error.
extern "C" int ggrms_bench_decode_native(const void* const* y, const void* const* gate,
                                         const float* const* w, void* const* out, int layers,
                                         int64_t width, int64_t group_size, float eps, int dtype,
                                         uint32_t flags, const ggrms_shape_t* shape,
                                         int bursts, int mode, double* dev_us, double* host_us) {
    if (layers <= 0 || bursts <= 0 || mode < 0 || mode > 5) return GGRMS_ERROR_INVALID_VALUE;
    ggrms_plan_t plan;
    const int st = ggrms_plan_tuned(y[0], gate[0], w[0], out[0], 1, width, group_size, width,
                                    width, width, eps, (ggrms_dtype_t)dtype, flags, shape, &plan);
    if (st != GGRMS_SUCCESS) return st;
    BurstRes r;
    if (hipStreamCreate(&r.s) != hipSuccess || hipEventCreate(&r.e0) != hipSuccess ||
        hipEventCreate(&r.e1) != hipSuccess)
        return -1;
    const bool empty = mode == 2 || mode == 3 || mode == 5;
    auto burst = [&]() -> int {
        for (int l = 0; l < layers; ++l) {
            if (empty) {
                if (ggrms_bench_empty(plan.workgroups, plan.block_threads, r.s) != 0) return -1;
            } else {
                const int rc = ggrms_forward_tuned(y[l], gate[l], w[l], out[l], 1, width,
                                                   group_size, width, width, width, eps,
                                                   (ggrms_dtype_t)dtype, flags, shape, r.s);
                if (rc != GGRMS_SUCCESS) return rc;
            }
        }
        return 0;
    };
    const bool graphed = mode == 1 || mode == 3 || mode >= 4;
    if (graphed) {
        if (hipStreamBeginCapture(r.s, hipStreamCaptureModeThreadLocal) != hipSuccess) return -1;
        const int rc = burst();
        const bool ended = hipStreamEndCapture(r.s, &r.graph) == hipSuccess;
        if (rc) return rc;
        if (!ended || hipGraphInstantiate(&r.exec, r.graph, nullptr, nullptr, 0) != hipSuccess)
            return -1;
    }
    auto run = [&]() -> int {
        if (graphed) return hipGraphLaunch(r.exec, r.s) == hipSuccess ? 0 : -1;
        return burst();
    };
    const auto t0 = std::chrono::steady_clock::now();
    while (std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count() < 0.1) {
        for (int i = 0; i < 8; ++i)
            if (const int rc = run()) return rc;
        if (hipStreamSynchronize(r.s) != hipSuccess) return -1;
    }
    std::vector<double> dev, host;
    if (mode >= 4) {
        for (int rep = 0; rep < 7; ++rep) {
            if (hipStreamSynchronize(r.s) != hipSuccess || hipEventRecord(r.e0, r.s) != hipSuccess)
                return -1;
            for (int b = 0; b < bursts; ++b)
                if (const int rc = run()) return rc;
            float ms = 0.0f;
            if (hipEventRecord(r.e1, r.s) != hipSuccess || hipEventSynchronize(r.e1) != hipSuccess ||
                hipEventElapsedTime(&ms, r.e0, r.e1) != hipSuccess)
                return -1;
            dev.push_back(ms * 1e3 / ((double)bursts * layers));
        }
        *dev_us = median_of(dev);
        *host_us = 0.0;
        return 0;
    }
    for (int b = 0; b < bursts; ++b) {
        if (hipStreamSynchronize(r.s) != hipSuccess || hipEventRecord(r.e0, r.s) != hipSuccess)
            return -1;
        const auto h0 = std::chrono::steady_clock::now();
        if (const int rc = run()) return rc;
        const auto h1 = std::chrono::steady_clock::now();
        float ms = 0.0f;
        if (hipEventRecord(r.e1, r.s) != hipSuccess || hipEventSynchronize(r.e1) != hipSuccess ||
            hipEventElapsedTime(&ms, r.e0, r.e1) != hipSuccess)
            return -1;
        dev.push_back(ms * 1e3 / layers);
        host.push_back(std::chrono::duration<double, std::micro>(h1 - h0).count() / layers);
    }
    *dev_us = median_of(dev);
    *host_us = median_of(host);
    return 0;
}

// Back-to-back launches of one job issued from C, so that a small job's
// per-launch figure is the GPU's and not the interpreter's: `launches`
// launches in a row, cycling over `sets` buffer sets (set i: y[i], gate[i],
// out[i]; one weight), timed between two events on a stream of its own, after
// about 100 ms of the same untimed; `bursts` such runs, median per launch.
// kind 0: ggrms_forward_tuned with `flags` / `shape` over [rows, width] views
// with the given row strides; kind 1: the plain two-read-one-write kernel over
// the same views, y[i] and gate[i] read, out[i] written (ggrms_bench_stream3
// over rows * width * element bytes per stream when all three are
// contiguous, ggrms_bench_stream3_rows over the strided rows otherwise).  Returns 0, a ggrms status, or -1 for
// a HIP error.
extern "C" int ggrms_bench_job_native(const void* const* y, const void* const* gate,
                                      const float* w, void* const* out, int sets, int64_t rows,
                                      int64_t width, int64_t group_size, int64_t y_row_stride,
                                      int64_t gate_row_stride, int64_t out_row_stride, float eps,
                                      int dtype, uint32_t flags, const ggrms_shape_t* shape,
                                      int kind, int launches, int bursts, double* dev_us) {
    if (sets <= 0 || launches <= 0 || bursts <= 0 || (kind != 0 && kind != 1))
        return GGRMS_ERROR_INVALID_VALUE;
    const int64_t esize = dtype == GGRMS_F32 ? 4 : 2;
    const int64_t nbytes = rows * width * esize;
    BurstRes r;
    if (hipStreamCreate(&r.s) != hipSuccess || hipEventCreate(&r.e0) != hipSuccess ||
        hipEventCreate(&r.e1) != hipSuccess)
        return -1;
    auto one = [&](int i) -> int {
        const int k = i % sets;
        if (kind == 1) {
            if (y_row_stride == width && gate_row_stride == width && out_row_stride == width)
                return ggrms_bench_stream3(y[k], gate[k], out[k], nbytes, r.s) ? -1 : 0;
            return ggrms_bench_stream3_rows(y[k], gate[k], out[k], rows, width * esize,
                                            y_row_stride * esize, gate_row_stride * esize,
                                            out_row_stride * esize, r.s)
                       ? -1
                       : 0;
        }
        return ggrms_forward_tuned(y[k], gate[k], w, out[k], rows, width, group_size, y_row_stride,
                                   gate_row_stride, out_row_stride, eps, (ggrms_dtype_t)dtype,
                                   flags, shape, r.s);
    };
    const auto t0 = std::chrono::steady_clock::now();
    int i = 0;
    while (std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count() < 0.1) {
        for (int j = 0; j < 64; ++j)
            if (const int rc = one(i++)) return rc;
        if (hipStreamSynchronize(r.s) != hipSuccess) return -1;
    }
    std::vector<double> dev;
    for (int b = 0; b < bursts; ++b) {
        if (hipStreamSynchronize(r.s) != hipSuccess || hipEventRecord(r.e0, r.s) != hipSuccess)
            return -1;
        for (int j = 0; j < launches; ++j)
            if (const int rc = one(i++)) return rc;
        float ms = 0.0f;
        if (hipEventRecord(r.e1, r.s) != hipSuccess || hipEventSynchronize(r.e1) != hipSuccess ||
            hipEventElapsedTime(&ms, r.e0, r.e1) != hipSuccess)
            return -1;
        dev.push_back(ms * 1e3 / launches);
    }
    *dev_us = median_of(dev);
    return 0;
}
